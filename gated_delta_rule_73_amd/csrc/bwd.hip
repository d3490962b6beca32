// Backward kernels of the chunked delta-rule operator (Delta family: DeltaNet, Gated DeltaNet).
//
// Per chunk, with dO the (scaled) output gradient and dW the gradient w.r.t. the memory at
// the chunk's end (reverse-mode of the chunk form used by the forward):
//   dR  = M^T dO + (e^{g_n-g} * K) dW^T
//   dW0 = e^{g_n} dW + dO^T (e^g * Q) - dR^T X          (carried to the previous chunk)
//   dQhat = dO W0,  dKbar = R dW,  dX = -dR W0,  dU = dR
//   dT = dU V^T + dX Khat^T,  dV = T^T dU,  dKhat = T^T dX
//   dL = -strictlower(L^-T (dT diag beta) L^-T),  dA = diag(beta) dL
//   dbeta_s = sum_t dT_ts Linv_ts + sum_s' dL_ss' A_ss'
//   Gram slots: dk += (dA*E) K + (dA*E)^T K + (dM*E)^T Q,  dq += (dM*E) K,  dM = tril(dO R^T)
// d log(alpha_t) collects every path through which log alpha_t scales a quantity.  Each
// such term carries the factor alpha_t itself, so it is summed directly (rectangle sums of
// the Gram pair terms over s < t <= u, suffix sums over u >= t, prefix sums over s < t)
// rather than as a difference of running sums; dividing by alpha_t then stays accurate
// even for strongly decaying tokens.
// Two launches: a sequential reverse scan per (sequence, head, value-row tile) that carries
// dW in float32 and records dW and dR per chunk, then a chunk-parallel kernel for the rest.
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

// ---------------------------------------------------------------------------------------
// Reverse scan over the chunks of one (sequence, head, value tile).
// ---------------------------------------------------------------------------------------
// Operands of one chunk of the reverse scan, held in registers while they are in flight.
// Gated DeltaNet-2 also needs the erase gates and beta (for a = beta e*k).
// Kimi Delta Attention reads Qhat = e^g Q and Kbar = e^{g_n-g} K (prepared per chunk) in
// place of Q and K, and the per-key-channel decay e^{g_n} of the rows this lane holds.
template <typename E, int D, int BV, int VAR>
struct BwdScanOps {
  RegTile<E, CH, D, 256> q, k, x;
  RegTile<E, CH, CH, 256> m;
  RegTile<E, CH, BV, 256> dO;
  float g;
  // gradient w.r.t. the residual output (used with RES): this lane's four columns of each
  // value tile of its chunk row, and beta of that row, both as loaded (from a valid row; masked
  // and converted where the step uses them, so the loads are never waited for early)
  typename VecT<4 * sizeof(E)>::type dr[BV / 16];
  E braw;
  // fused q/k normalisation: 1 / ||q|| of the dO rows this lane holds, 1 / ||k|| of dR^T's
  // chunk row 16 w + lrow
  float rnq[RegTile<E, CH, BV, 256>::IT], rnk;
};
template <typename E, int D, int BV>
struct BwdScanOps<E, D, BV, VAR_GDN2> {
  RegTile<E, CH, D, 256> q, k, x, e;
  RegTile<E, CH, CH, 256> m;
  RegTile<E, CH, BV, 256> dO;
  float g;
  uint32_t braw2;  // beta of this lane's token as loaded (0 if absent or past the end)
  // fused q/k normalisation: 1 / ||q|| of the dO rows this lane holds, 1 / ||k|| of its token
  float rnq[RegTile<E, CH, BV, 256>::IT], rnk;
};
template <typename E, int D, int BV>
struct BwdScanOps<E, D, BV, VAR_GDN2L> : BwdScanOps<E, D, BV, VAR_GDN2> {};
template <typename E, int D, int BV>
struct BwdScanOps<E, D, BV, VAR_KDA> {
  RegTile<E, CH, D, 256> q, k, x;
  RegTile<E, CH, CH, 256> m;
  RegTile<E, CH, BV, 256> dO;
  f32x4 eg[D / 64];
  typename VecT<4 * sizeof(E)>::type dr[BV / 16];  // as in the general case (RES)
  E braw;
};
template <typename E, int D, int BV>
struct BwdScanOps<E, D, BV, VAR_GLA> {  // nothing erased: no X
  RegTile<E, CH, D, 256> q, k;
  RegTile<E, CH, CH, 256> m;
  RegTile<E, CH, BV, 256> dO;
  f32x4 eg[D / 64];
};

// RES (delta family, Kimi Delta Attention): the residual r_t = R_t / beta_t was an output too; its gradient dr adds
// dr_t / beta_t to dR_t before dR feeds the memory gradient and the chunk kernel.  dRog, if not
// NULL, also receives dR without that term (the beta gradient is formed from it, see
// k_bwd_res_dbeta).
// QKN (delta family, Gated DeltaNet-2): q and k are normalised to unit length per token.  The
// raw rows are read and the preparation's factors Rng (1 / ||q||, 1 / ||k|| per unit) are
// applied to the rows that meet them: to scale e^g dO in the update Q^T (e^g dO), to
// e^{g_n-g} (dW K^T) in dR.  Gated DeltaNet-2 folds 1 / ||k_t|| into beta_t of its erase
// direction a = beta e*k, the only product its keys enter here.
template <typename E, int D, int BV, int VAR, bool RES, bool QKN>
__global__ __launch_bounds__(256) void k_bwd_scan(Geo geo, ScanSeg sg, const E* __restrict__ q, const E* __restrict__ k,
                                                  const E* __restrict__ dO, const E* __restrict__ Xg,
                                                  const E* __restrict__ Mg, const float* __restrict__ Gg,
                                                  const float* __restrict__ dht, E* __restrict__ dHs,
                                                  E* __restrict__ dRg, float* __restrict__ dh0,
                                                  const E* __restrict__ beta, const E* __restrict__ erase,
                                                  const E* __restrict__ drin, E* __restrict__ dRog,
                                                  const float* __restrict__ Rng) {
  GDR_POISON_ALL();
  constexpr int NT = 256, LD = D + pad16<E>(), LDV = BV + pad16<E>(), LDR = CH + pad16<E>();
  constexpr int NJ = D / 64, NI = BV / 16;
  constexpr bool G2 = VAR == VAR_GDN2 || VAR == VAR_GDN2L;
  constexpr bool G2L = VAR == VAR_GDN2L;  // its gates are logits
  constexpr bool KDA = VAR == VAR_KDA || VAR == VAR_GLA;  // decay per key channel, per-unit operands
  constexpr bool NOX = VAR == VAR_GLA;  // nothing erased: X = 0, no dR^T X term
  constexpr bool DEC = VAR == VAR_GATED || G2;  // scalar decay
  static_assert(!RES || VAR == VAR_DELTANET || VAR == VAR_GATED || VAR == VAR_KDA, "residual gradient: not GDN-2, GLA");
  static_assert(!QKN || (VAR != VAR_KDA && VAR != VAR_GLA), "fused q/k normalisation: not the per-unit operands");
  __shared__ __align__(16) E As[G2 ? CH * LD : 8];  // a = beta e*k (GDN-2)
  __shared__ float bsh[CH];
  __shared__ float rks[QKN && (VAR == VAR_GDN2 || VAR == VAR_GDN2L) ? CH : 1];  // Gated DeltaNet-2: 1 / ||k_t||
  __shared__ __align__(16) E Qs[CH * LD];
  __shared__ __align__(16) E Ks[CH * LD];
  __shared__ __align__(16) E Xs[VAR == VAR_GLA ? 8 : CH * LD];
  __shared__ __align__(16) E Ms[CH * LDR];
  // scale * dO and scale * e^g * dO, row-major, read through transposing reads; for bfloat16,
  // rows 64 bytes apart keep those reads free of bank conflicts
  constexpr int LDO = std::is_same<E, float>::value ? BV + 4 : 32;
  static_assert(LDO >= BV, "a dO row fits");
  __shared__ __align__(16) E dOt[CH * LDO];
  __shared__ __align__(16) E dOg[CH * LDO];
  __shared__ __align__(16) E dWs[BV * LD];
  __shared__ __align__(16) E dRt[CH * LDO];   // -dR, row-major, read like dO
  __shared__ __align__(16) E dRn[CH * LDV];   // dR
  __shared__ __align__(16) E dRo[RES ? CH * LDV : 8];  // dR without the residual's term
  __shared__ float gs[CH];

  constexpr int NVR = D / BV;
  int sq, h, vt;
  if (!scan_block(geo, sg.mode == 1 ? 2 * NVR : NVR, sq, h, vt)) return;
  const bool virt = vt >= NVR;  // mode 1: rows of the segment's linear part (no dO term)
  const int i0 = (virt ? vt - NVR : vt) * BV;
  const SeqPos sp = seq_pos(geo, sq);
  const int w = wave_id();
  const long mem = (long)sq * geo.H + h;
  const long sbase = mem * D;
  const int nsg = sg.mode != 0 ? seg_count(sg, sp.nchunks) : 1;
  const int seg = sg.mode == 3 ? nsg - 1 - sg.part : (int)blockIdx.y;
  int c0 = 0, c1 = sp.nchunks;
  if (sg.mode != 0) {
    if (seg < 0 || seg >= nsg) return;  // mode 3: this sequence has no such part
    if (sg.mode == 1 && seg == 0) return;  // walked in reverse, the first segment's map is never applied
    c0 = seg * sg.lseg;
    c1 = min(sp.nchunks, c0 + sg.lseg);
  }
  const bool snap = sg.mode != 1;  // record dW and dR per chunk
  const float* init = nullptr;      // memory gradient at the end of the covered chunks
  if (sg.mode == 2) init = sg.starts + (mem * sg.max_seg + seg) * D * D;
  else if (sg.mode == 3) init = seg == nsg - 1 ? (dht ? dht + sbase * D : nullptr) : sg.maps + (mem * sg.max_seg + seg) * D * D;
  else if (sg.mode == 0 && dht) init = dht + sbase * D;

  f32x4 S[NJ][NI];  // dW^T tiles
#pragma unroll
  for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int j0 = acc_row(16 * (w + 4 * qq), 0), i = i0 + acc_col(16 * it);
      if (init) {
        const float4 x = *reinterpret_cast<const float4*>(init + (long)i * D + j0);
        S[qq][it] = f32x4{x.x, x.y, x.z, x.w};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[qq][it][r] = (virt && j0 + r == i) ? 1.f : 0.f;
      }
    }

  // Chunk c - 2 is loaded while chunk c is computed (two register sets, loop unrolled by two).
  // Loads before the first chunk repeat it, so every step issues the same memory operations.
  // The loads of a step are issued in two parts (part < 0: all), each in a stretch of matrix-
  // core work that hides its issue: X, M and dO with dR, the queries, keys and gates with the
  // update of dW.
  using Ops = BwdScanOps<E, D, BV, VAR>;
  auto load = [&](Ops& p, int c, int part) {
    const int cc = max(c, c0);
    const long u = (long)(sp.gc0 + cc) * geo.H + h;
    const int n = min(CH, sp.len - cc * CH);
    const long tk = tok_index(geo, sp.b, h, sp.bos + cc * CH);
    if (part <= 0) {
      if constexpr (QKN) {  // first, so that the step's waits for them wait for little else
        load_row_factors(p.dO, Rng + u * 2 * CH, p.rnq);
        p.rnk = Rng[u * 2 * CH + CH + (G2 ? (int)(threadIdx.x & (CH - 1)) : 16 * w + lrow())];
      }
      if constexpr (!NOX) p.x.load(Xg + u * CH * D, D, CH);
      p.m.load(Mg + u * CH * CH, CH, CH);
      p.dO.load(dO + tk * D + i0, D, n);
    }
    if (part != 0) {
      if constexpr (KDA) {
        p.q.load(q + u * CH * D, D, CH);
        p.k.load(k + u * CH * D, D, CH);
#pragma unroll
        for (int qq = 0; qq < NJ; ++qq) p.eg[qq] = *reinterpret_cast<const f32x4*>(Gg + u * D + acc_row(16 * (w + 4 * qq), 0));
      } else {
        p.q.load(q + tk * D, D, n);
        p.k.load(k + tk * D, D, n);
        p.g = Gg[u * CH + (threadIdx.x & (CH - 1))];
      }
      if constexpr (RES) {  // accumulator layout of dR^T: row 16 w + lrow, columns 16 it + 4 lgrp
        const int t = min(16 * w + lrow(), n - 1);
        p.braw = beta[tk + t];
#pragma unroll
        for (int it = 0; it < NI; ++it)
          p.dr[it] = *reinterpret_cast<const typename VecT<4 * sizeof(E)>::type*>(drin + (tk + t) * D + i0 + 16 * it +
                                                                                 4 * lgrp());
      }
      if constexpr (G2) {
        p.e.load(erase + tk * D, D, n);
        p.braw2 = load_gate_raw(beta ? beta + tk : nullptr, n, (int)(threadIdx.x & (CH - 1)));
      }
    }
  };
  auto step = [&](int c, Ops& p) {
    const long u = (long)(sp.gc0 + c) * geo.H + h;
    [[maybe_unused]] const int n = min(CH, sp.len - c * CH);
    float rnk_c = 0.f;  // this chunk's key factor, kept before p is refilled (the dO rows' are used first)
    if constexpr (QKN) rnk_c = p.rnk;
    p.q.store(Qs, LD);
    p.k.store(Ks, LD);
    if constexpr (!NOX) p.x.store(Xs, LD);
    p.m.store(Ms, LDR);
    f32x4 egk[NJ];  // KDA: this chunk's per-row decay, kept before p is refilled
    if constexpr (KDA) {
#pragma unroll
      for (int qq = 0; qq < NJ; ++qq) egk[qq] = p.eg[qq];
    } else {
      if (threadIdx.x < CH) gs[threadIdx.x] = p.g;
    }
    if constexpr (G2) {
      if (threadIdx.x < CH)  // beta (1 when absent), 0 past the end; converted here, where it is used
        bsh[threadIdx.x] = ((int)threadIdx.x < n) ? (beta ? g2_gate<G2L>(gate_from_raw<E>(p.braw2)) : 1.f) : 0.f;
      if constexpr (QKN) {
        if (threadIdx.x < CH) rks[threadIdx.x] = rnk_c;
      }
    }
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) store4_t(dWs, LD, 16 * (w + 4 * qq), 16 * it, S[qq][it]);
    __syncthreads();
    // dO tile twice, plain and with e^{g_t} (rows t >= n are zero), one vector store each
    {
      using RT = RegTile<E, CH, BV, NT>;
#pragma unroll
      for (int it = 0; it < RT::IT; ++it) {
        if (RT::TOTAL % NT == 0 || threadIdx.x + it * NT < RT::TOTAL) {
          const int t = p.dO.row(it), i = p.dO.col(it);
          const E* e = reinterpret_cast<const E*>(&p.dO.v[it]);
          float eg = 1.f;  // e^{g_t} (times 1 / ||q_t||: the update meets the raw q_t)
          if constexpr (DEC) eg = __expf(gs[t]);
          if constexpr (QKN) eg *= p.rnq[it];
          typename RT::V pv, gv;
          E* pe = reinterpret_cast<E*>(&pv);
          E* ge = reinterpret_cast<E*>(&gv);
#pragma unroll
          for (int x = 0; x < RT::VE; ++x) {
            const float val = virt ? 0.f : geo.scale * (float)e[x];
            pe[x] = (E)val;
            ge[x] = (E)(val * eg);
          }
          *reinterpret_cast<typename RT::V*>(dOt + t * LDO + i) = pv;
          *reinterpret_cast<typename RT::V*>(dOg + t * LDO + i) = gv;
        }
      }
    }
    if constexpr (G2) {
      using RE = decltype(p.e);
#pragma unroll
      for (int it = 0; it < RE::IT; ++it) {  // one vector store per register vector
        const int t = p.e.row(it), j0 = p.e.col(it);
        float bt = bsh[t];
        if constexpr (QKN) bt *= rks[t];  // the raw k_t scaled to unit length
        typename RE::V av;
        E* ae = reinterpret_cast<E*>(&av);
#pragma unroll
        for (int x = 0; x < RE::VE; ++x) ae[x] = (E)(bt * g2_gate<G2L>((float)p.e.elem(it, x)) * (float)p.k.elem(it, x));
        *reinterpret_cast<typename RE::V*>(As + t * LD + j0) = av;
      }
    }
    if (snap) s2g_full<E, BV, D, NT>(dHs + u * D * D + (long)i0 * D, D, dWs, LD);
    __syncthreads();
    load(p, c - 2, 0);
    const float gn = gs[CH - 1];
    // dR^T: the lane holds chunk row tl and four consecutive value columns
    const int tl = 16 * w + lrow();
    float dec = 1.f;  // e^{g_n - g_t} (times 1 / ||k_t||: dW meets the raw k_t)
    if constexpr (DEC) dec = __expf(gn - gs[tl]);
    if constexpr (QKN && !G2) dec *= rnk_c;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const f32x4 a1 = mma_k<E, CH>(zero4(), colk(dOt, LDO), 16 * it, colk(Ms, LDR), 16 * w);
      const f32x4 a2 = mma_k<E, D>(zero4(), rowk(dWs, LD), 16 * it, rowk(G2 ? As : Ks, LD), 16 * w);
      f32x4 dr = a1 + dec * a2;
      const int c4 = 16 * it + 4 * lgrp();
      if constexpr (RES) {  // + dr / beta for the rows of this chunk (none for the linear part)
        put4(dRo + tl * LDV + c4, dr);
        const bool ok = tl < n && !virt;
        const float binv = ok ? 1.f / (float)p.braw : 0.f;
        const E* x = reinterpret_cast<const E*>(&p.dr[it]);
        dr += binv * f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
      }
      put4(dRt + tl * LDO + c4, -dr);
      put4(dRn + tl * LDV + c4, dr);
    }
    __syncthreads();
    if (snap) {
      s2g_full<E, CH, BV, NT>(dRg + u * CH * D + i0, D, dRn, LDV);
      if constexpr (RES) {
        if (dRog) s2g_full<E, CH, BV, NT>(dRog + u * CH * D + i0, D, dRo, LDV);
      }
    }
    load(p, c - 2, 1);
    float eg = 1.f;
    if constexpr (DEC) eg = __expf(gn);
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        if constexpr (KDA) S[qq][it] *= egk[qq];
        else S[qq][it] *= eg;
        S[qq][it] = mma_k<E, CH>(S[qq][it], colk(Qs, LD), 16 * (w + 4 * qq), colk(dOg, LDO), 16 * it);
        if constexpr (!NOX) S[qq][it] = mma_k<E, CH>(S[qq][it], colk(Xs, LD), 16 * (w + 4 * qq), colk(dRt, LDO), 16 * it);
      }
    __syncthreads();
    GDR_POISON_ALL();  // debug builds: nothing in LDS is carried to the next step
  };
  if (c1 > c0) {
    Ops pa, pb;
    load(pa, c1 - 1, -1);
    load(pb, c1 - 2, -1);
    // Every trip of the loop runs both steps (an odd first chunk runs after it), so the
    // memory operations in flight at the top of the loop are the same on every path.
    int c = c1 - 1;
    for (; c - 1 >= c0; c -= 2) {
      step(c, pa);
      step(c - 1, pb);
    }
    if (c >= c0) step(c, pa);
  }
  float* out = nullptr;  // dh0, this segment's map, or (mode 3) the next part's start
  if (sg.mode == 1) out = sg.maps + ((mem * sg.max_seg + seg) * 2 + (virt ? 1 : 0)) * D * D;
  else if (sg.mode == 3 && seg > 0) out = sg.maps + (mem * sg.max_seg + seg - 1) * D * D;
  else if (dh0 && seg == 0) out = dh0 + sbase * D;
  if (out) {
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int j0 = acc_row(16 * (w + 4 * qq), 0), i = i0 + acc_col(16 * it);
        const f32x4 x = S[qq][it];
        *reinterpret_cast<float4*>(out + (long)i * D + j0) = make_float4(x[0], x[1], x[2], x[3]);
      }
  }
}

// ---------------------------------------------------------------------------------------
// Chunk-local gradients: per (head, chunk), 512 threads, LDS regions reused across phases.
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct BwdLds {
  static constexpr int LD = D + pad16<E>(), LDR = CH + pad16<E>(), LF = CH + 4;
  static constexpr int TK = CH * LD * (int)sizeof(E);   // 64 x D token tile
  static constexpr int TH = CH * LD * (int)sizeof(E);  // 64 value rows of the memory
  static constexpr int SQ = CH * LDR * (int)sizeof(E);  // 64 x 64 in E
  static constexpr int F = CH * LF * 4;                 // 64 x 64 float
  static constexpr int oK = 0, odR = TK, odX = 2 * TK, odM = 3 * TK, oU = 3 * TK + SQ;
  // phase 1 (state part)
  static constexpr int odO = oU, oR = oU + TK, oWh = oU + 2 * TK, odWh = oU + 2 * TK + TH;
  static constexpr int endP1 = oU + 2 * TK + 2 * TH;
  // phase 2 (WY part) and 3 (Gram part)
  static constexpr int oA = oU, odT = oU + F, oLi = oU + 2 * F, oVP = oU + 3 * F;
  static constexpr int endVP = oU + 3 * F + (TK > F ? TK : F);
  // (dT diag(beta)) Linv^T: in the dX region when a 64 x 64 float tile fits there
  static constexpr int oPt = TK >= F ? odX : endVP;
  static constexpr int endP2 = TK >= F ? endVP : endVP + F;
  static constexpr int oQ = oLi, oPair = oVP, oAt = odR, oMt = odR + SQ;
  // bfloat16 copies of L^{-1} and T = L^{-1} diag(beta) as matrix-core operands (the float32
  // path reads L^{-1} directly)
  static constexpr bool BCOPY = !std::is_same<E, float>::value;
  static constexpr int BIG0 = endP1 > endP2 ? endP1 : endP2;
  static constexpr int oLb = BIG0, oTb = BIG0 + SQ;
  static constexpr int BIG = BIG0 + (BCOPY ? 2 * SQ : 0);
  static_assert(TK <= F, "Q must fit the region of Linv");
  static_assert(2 * SQ <= 2 * TK, "Gram operand buffers must fit the dR/dX regions");
};


// RES: the residual r = R / beta was an output; dbeta gains -(dr . r) / beta = -(dr . R) / beta^2.
// LOG: beta and alpha are logits x; the gradients returned are w.r.t. x:
// dx_beta = dbeta beta (1 - beta), dx_alpha = d log(alpha) * (-sigmoid(x_alpha)).
// QKN: q and k are normalised per token, x~ = x / ||x||: the raw rows are read and scaled by
// the preparation's factors rn = 1/||x|| (Rng) as the preparation scaled them, and dq, dk are
// returned w.r.t. the raw rows: dx = (dx~ - x~ (x~ . dx~)) / ||x||, formed in float32 before the
// gradients are rounded.
template <typename E, int D, int VAR, bool RES, bool LOG, bool QKN>
__global__ __launch_bounds__(512) void k_bwd_chunk(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                   const E* __restrict__ v, const E* __restrict__ beta,
                                                   const E* __restrict__ alpha, const E* __restrict__ dO,
                                                   const E* __restrict__ Mg, const float* __restrict__ Gg,
                                                   const E* __restrict__ Hs, const E* __restrict__ Rg,
                                                   const E* __restrict__ dHs, const E* __restrict__ dRg,
                                                   const float* __restrict__ Lig,
                                                   E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
                                                   E* __restrict__ dbeta, E* __restrict__ dalpha,
                                                   const E* __restrict__ drin, const float* __restrict__ Rng,
                                                   int ts_part, int ts_lseg) {
  GDR_POISON_ALL();
  using Ly = BwdLds<E, D>;
  constexpr int NT = 512, LD = Ly::LD, LDR = Ly::LDR, LF = Ly::LF;
  constexpr int KH = 64, NH = D / KH;  // the memory is read in blocks of 64 value rows
  constexpr int NQ = D / 32;           // 64 x D tiles per wave when all 8 waves share a matrix
  constexpr bool GATED = VAR == VAR_GATED;
  __shared__ __align__(16) char smem[Ly::BIG];
  __shared__ __align__(16) float gs[CH], bs[CH], red[NT / 64];
  __shared__ float part8[NT / CH][CH], pdb[CH], part8c[NT / CH][CH];  // partial sums
  __shared__ float rq[4][CH], rkh[8][CH], rkb[8][CH];
  __shared__ float rkn[QKN ? 8 : 1][CH];  // QKN: k~ . dk~ per row, the part of each wave
  __shared__ float rdr[RES ? CH : 1];  // dr_t . R_t (residual output)
  __shared__ float invq[QKN ? CH : 1], invk[QKN ? CH : 1];  // 1 / ||x|| of the rows of q and k

  E* Ks = reinterpret_cast<E*>(smem + Ly::oK);
  E* dRs = reinterpret_cast<E*>(smem + Ly::odR);
  E* dXs = reinterpret_cast<E*>(smem + Ly::odX);
  E* dMs = reinterpret_cast<E*>(smem + Ly::odM);

  // ts_lseg > 0: blocks (c, head, sequence) cover the chunks of part ts_part of every sequence,
  // its segment nseg - 1 - ts_part of ts_lseg chunks (as the reverse scan's mode 3 counts them)
  int gc = blockIdx.x;
  if (ts_lseg > 0) {
    const SeqPos sp = seq_pos(geo, blockIdx.z);
    const int seg = max(1, (sp.nchunks + ts_lseg - 1) / ts_lseg) - 1 - ts_part;
    const int c = seg * ts_lseg + (int)blockIdx.x;
    if (seg < 0 || c >= sp.nchunks) return;
    gc = sp.gc0 + c;
  }
  const int h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wm = w & 3, wn = w >> 2;
  const int n = cp.n;

  // ================= phase 1: products with the memory W0 and its gradient dW
  f32x4 acc1[D / 16];  // waves 0-3: (dO W0)^T = dQhat^T; waves 4-7: (dR W0)^T; both column
                       // tile wm (stored four columns at a time)
  f32x4 dka[NQ];       // dk, held transposed: row t = 16 wm + lrow, four consecutive columns
                       // of column tiles wn*NQ + qq
  f32x4 acc3[2];       // dM tiles w and w + 8
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc1[i] = zero4();
#pragma unroll
  for (int i = 0; i < NQ; ++i) dka[i] = zero4();
  acc3[0] = acc3[1] = zero4();
  float gam = 0.f;
  RegTile<E, KH, D, NT> pW, pdW;      // one 64-row block of W0 and of dW, next block prefetched
  RegTile<E, CH, D, NT> pV, pQ;       // V and Q, used in later phases
  RegTile<E, CH, CH, NT> pM;          // M, used for the decay gradient
  RegTile<float, CH, CH, NT> pLi;     // the forward's L^{-1}, used in phase 2
  float rnq[decltype(pQ)::IT];        // QKN: 1 / ||q|| of the rows of pQ this thread holds
  // The per-token decay and beta are loaded before the tiles and staged after the first tile
  // stores: waiting for them then waits for nothing else, where loaded after the tiles they
  // would make the staging wait for every tile in flight (the wait counters are ordered).
  float graw = 0.f, iqraw = 0.f, ikraw = 0.f;  // iqraw, ikraw: 1 / ||q||, 1 / ||k|| (QKN)
  E braw = E(0.f), araw = E(1.f);  // araw: alpha (or its logit) of this lane's token, for the end
  if (threadIdx.x < CH) {
    graw = Gg[u * CH + threadIdx.x];
    braw = beta[tk + min((int)threadIdx.x, n - 1)];
    if constexpr (GATED) araw = alpha[tk + min((int)threadIdx.x, n - 1)];
    if constexpr (QKN) {
      iqraw = Rng[u * 2 * CH + threadIdx.x];
      ikraw = Rng[u * 2 * CH + CH + threadIdx.x];
    }
  }
  {
    E* dOs = reinterpret_cast<E*>(smem + Ly::odO);
    E* Rs = reinterpret_cast<E*>(smem + Ly::oR);
    E* Wh = reinterpret_cast<E*>(smem + Ly::oWh);
    E* dWh = reinterpret_cast<E*>(smem + Ly::odWh);
    {
      RegTile<E, CH, D, NT> r0, r1, r2, r3;
      // QKN: the factors of the rows this thread holds, loaded first (the waits are ordered:
      // loaded after the tiles, scaling K would wait for every tile in flight)
      float rnk[decltype(r0)::IT];
      if constexpr (QKN) {
        load_row_factors(pQ, Rng + u * 2 * CH, rnq);
        load_row_factors(r0, Rng + u * 2 * CH + CH, rnk);
      }
      r0.load(k + tk * D, D, n);
      r1.load(dO + tk * D, D, n);
      r2.load(Rg + u * CH * D, D, CH);
      r3.load(dRg + u * CH * D, D, CH);
      pW.load(Hs + u * D * D, D, KH);
      pdW.load(dHs + u * D * D, D, KH);
      pV.load(v + tk * D, D, n);
      pQ.load(q + tk * D, D, n);
      pM.load(Mg + u * CH * CH, CH, CH);
      pLi.load(Lig + u * CH * CH, CH, CH);
      if constexpr (QKN) scale_rows(r0, rnk);
      if constexpr (RES) {  // dr_t . R_t per row, from the registers: a row is VPR adjacent lanes
        RegTile<E, CH, D, NT> rd;
        rd.load(drin + tk * D, D, n);
        using RT = decltype(rd);
        static_assert(RT::TOTAL % NT == 0 && 64 % RT::VPR == 0, "whole rows per lane group");
#pragma unroll
        for (int it = 0; it < RT::IT; ++it) {
          float a = 0.f;
#pragma unroll
          for (int x = 0; x < RT::VE; ++x) a += (float)r2.elem(it, x) * (float)rd.elem(it, x);
#pragma unroll
          for (int off = RT::VPR / 2; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
          if (threadIdx.x % RT::VPR == 0) rdr[rd.row(it)] = a;
        }
      }
      r0.store(Ks, LD);
      r1.store(dOs, LD);
      r2.store(Rs, LD);
      r3.store(dRs, LD);
    }
    if (threadIdx.x < CH) {
      const int t = threadIdx.x;
      gs[t] = graw;
      bs[t] = (t < n) ? (LOG ? gate_sigmoid((float)braw) : (float)braw) : 0.f;
      if constexpr (QKN) {
        invq[t] = iqraw;
        invk[t] = ikraw;
      }
    }
    for (int ih = 0; ih < NH; ++ih) {
      __syncthreads();
      pW.store(Wh, LD);  // rows i (value), columns j (key): read k-major below
      pdW.store(dWh, LD);
      if constexpr (GATED) {  // <W0, dW> over this block of rows, from the registers
#pragma unroll
        for (int it = 0; it < decltype(pW)::IT; ++it)
#pragma unroll
          for (int x = 0; x < decltype(pW)::VE; ++x) gam += (float)pW.elem(it, x) * (float)pdW.elem(it, x);
      }
      if (ih + 1 < NH) {
        pW.load(Hs + u * D * D + (long)(ih + 1) * KH * D, D, KH);
        pdW.load(dHs + u * D * D + (long)(ih + 1) * KH * D, D, KH);
      }
      __syncthreads();
      if (w < 4) {
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = mma_k<E, KH>(acc1[nt], colk(Wh, LD), 16 * nt, rowk(dOs + ih * KH, LD), 16 * wm);
      } else {
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = mma_k<E, KH>(acc1[nt], colk(Wh, LD), 16 * nt, rowk(dRs + ih * KH, LD), 16 * wm);
      }
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
        dka[qq] = mma_k<E, KH>(dka[qq], colk(dWh, LD), 16 * (wn * NQ + qq), rowk(Rs + ih * KH, LD), 16 * wm);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int id = w + 8 * e;
        acc3[e] = mma_k<E, KH>(acc3[e], rowk(Rs + ih * KH, LD), 16 * (id & 3), rowk(dOs + ih * KH, LD), 16 * (id >> 2));  // dM^T
      }
    }
  }
  const float gn = gs[CH - 1];
  // e^{g_t}, e^{g_n - g_t} for the row t of the transposed dq and dk tiles this lane holds
  const int tr = 16 * wm + lrow();
  float egt = 1.f, egdt = 1.f;
  if constexpr (GATED) {
    egt = __expf(gs[tr]);
    egdt = __expf(gn - gs[tr]);
  }
  // dq (first term) stays in acc1 for waves 0-3; dX goes to LDS from waves 4-7
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    if (w < 4) {
      acc1[nt] *= geo.scale * egt;
    } else {
      store4_t(dXs, LD, 16 * nt, 16 * wm, -acc1[nt]);
    }
  }
  // dk (first term): e^{g_n - g_t} dKbar, and the rows' Kbar . dKbar
  {
    float part = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      dka[qq] *= egdt;
      const f32x4 kv = get4(Ks + tr * LD + 16 * (wn * NQ + qq) + 4 * lgrp());
      part += kv[0] * dka[qq][0] + kv[1] * dka[qq][1] + kv[2] * dka[qq][2] + kv[3] * dka[qq][3];
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rkb[w][tr] = part;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;  // dM tile (rows mt, columns nt), held transposed
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (acc_row(16 * nt, r) <= acc_col(16 * mt)) ? geo.scale * acc3[e][r] : 0.f;
    store4_t(dMs, LDR, 16 * nt, 16 * mt, x);
  }
  if constexpr (GATED) {
    gam = wave_sum(gam);
    if (lane_id() == 0) red[w] = gam;
  }
  __syncthreads();
  GDR_POISON(smem + Ly::oU, Ly::endP1 - Ly::oU);  // dO, R and the memory blocks are no longer read

  // ================= phase 2: the WY / triangular-solve part
  float* As = reinterpret_cast<float*>(smem + Ly::oA);
  float* dTs = reinterpret_cast<float*>(smem + Ly::odT);
  float* Li = reinterpret_cast<float*>(smem + Ly::oLi);
  E* Vs = reinterpret_cast<E*>(smem + Ly::oVP);
  pV.store(Vs, LD);
  pLi.store(Li, LF);  // L^{-1} as the forward computed it
  // A (strictly lower) formed again from K as the forward formed it (the same products of the
  // same operands, so the same values): 16 KiB less to write forward and to read here
#pragma unroll
  for (int jr = 0; jr < 2; ++jr) {  // ten tiles: waves 0 and 1 take a second one
    const int job = w + jr * (NT / 64);
    if (job >= 10) break;
    int mt, nt;
    tri_tile(job, mt, nt);
    const f32x4 acc = mma_k<E, D>(zero4(), rowk(Ks, LD), 16 * nt, rowk(Ks, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    float val[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sc = s0 + r;
      float dec = 1.f;
      if constexpr (GATED) dec = __expf(gs[t] - gs[sc]);
      val[r] = sc < t ? acc[r] * dec : 0.f;
    }
    *reinterpret_cast<float4*>(As + t * LF + s0) = make_float4(val[0], val[1], val[2], val[3]);
  }
#pragma unroll
  for (int i = 0; i < CH * CH / 4 / NT; ++i) {  // tiles above the diagonal
    const int idx = threadIdx.x + i * NT, t = idx >> 4, s0 = (idx & 15) * 4;
    if ((s0 >> 4) > (t >> 4)) *reinterpret_cast<float4*>(As + t * LF + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  E* Lb = reinterpret_cast<E*>(smem + Ly::oLb);
  E* Tb = reinterpret_cast<E*>(smem + Ly::oTb);
  if constexpr (Ly::BCOPY) {  // from the registers: L^{-1} and L^{-1} diag(beta) in bfloat16
    using RL = decltype(pLi);
    static_assert(RL::VE == 4, "four floats per vector");
#pragma unroll
    for (int it = 0; it < RL::IT; ++it) {
      const int t = pLi.row(it), s0 = pLi.col(it);
      const f32x4 l = {pLi.elem(it, 0), pLi.elem(it, 1), pLi.elem(it, 2), pLi.elem(it, 3)};
      const float4 b4 = *reinterpret_cast<const float4*>(bs + s0);
      put4(Lb + t * LDR + s0, l);
      put4(Tb + t * LDR + s0, l * f32x4{b4.x, b4.y, b4.z, b4.w});
    }
  }
  // operand views of L^{-1} (rows t, columns s) and of T^T
  const auto LiRow = [&]() { if constexpr (Ly::BCOPY) return rowk(Lb, LDR); else return rowk(Li, LF); }();
  const auto LiCol = [&]() { if constexpr (Ly::BCOPY) return colk(Lb, LDR); else return colk(Li, LF); }();
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
    const f32x4 a = mma_k<E, D>(zero4(), rowk(dRs, LD), 16 * mt, rowk(Vs, LD), 16 * nt);
    const f32x4 b = mma_k<E, D>(zero4(), rowk(dXs, LD), 16 * mt, rowk(Ks, LD), 16 * nt);
    const int s = acc_col(16 * nt);
    float es = 1.f;
    if constexpr (GATED) es = __expf(gs[s]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = acc_row(16 * mt, r);
      dTs[t * LF + s] = (s <= t) ? a[r] + b[r] * es : 0.f;
    }
  }
  // dV = T^T dR and dKhat = T^T dX with T = Linv diag(beta)
  const auto Tt = [&]() { if constexpr (Ly::BCOPY) return colk(Tb, LDR); else return TtView{Li, LF, bs}; }();
  f32x4 dva[NQ];
  {
    float part = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int nt = wn * NQ + qq;
      dva[qq] = mma_k<E, CH>(zero4(), colk(dRs, LD), 16 * nt, Tt, 16 * wm);  // dV^T
      const f32x4 kh = egt * mma_k<E, CH>(zero4(), colk(dXs, LD), 16 * nt, Tt, 16 * wm);  // dKhat^T
      const f32x4 kv = get4(Ks + tr * LD + 16 * nt + 4 * lgrp());
      part += kv[0] * kh[0] + kv[1] * kh[1] + kv[2] * kh[2] + kv[3] * kh[3];
      dka[qq] += kh;
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rkh[w][tr] = part;
  }
  __syncthreads();
  GDR_POISON(dXs, Ly::TK);  // dX, dR and V are no longer read
  GDR_POISON(dRs, Ly::TK);
  GDR_POISON(smem + Ly::oVP, Ly::endVP - Ly::oVP);
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) store4_t(Vs, LD, 16 * (wn * NQ + qq), 16 * wm, dva[qq]);
  {  // dbeta from T = Linv diag(beta): column sums, eight threads per column
    const int s = threadIdx.x & (CH - 1), pt = threadIdx.x >> 6;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < CH / (NT / CH); ++i) a += dTs[(pt + i * (NT / CH)) * LF + s] * Li[(pt + i * (NT / CH)) * LF + s];
    part8c[pt][s] = a;  // summed when dbeta is written
  }
  __syncthreads();
  s2g_rows<E, CH, D, NT>(dv + tk * D, D, Vs, LD, n);
  // gradient w.r.t. Linv is dT diag(beta); Pt = (dT diag(beta)) Linv^T, staged where dX was
  // (free once dT and dKhat have been formed) or in a region of its own
  float* Pt = reinterpret_cast<float*>(smem + Ly::oPt);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
    const f32x4 acc = mma_k<E, CH>(zero4(), RowKScaled{dTs, LF, bs}, 16 * mt, LiRow, 16 * nt);
    store4_t(Pt, LF, 16 * mt, 16 * nt, acc);
  }
  __syncthreads();
  GDR_POISON(smem + Ly::oVP, Ly::endVP - Ly::oVP);  // dV has been written out
  // dL (strictly lower); dT is no longer read, so dL overwrites it in place
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
    const f32x4 acc = mma_k<E, CH>(zero4(), LiCol, 16 * mt, rowk(Pt, LF), 16 * nt);
    f32x4 dl;
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[r] = (acc_col(16 * nt) < acc_row(16 * mt, r)) ? -acc[r] : 0.f;
    store4_n(dTs, LF, 16 * mt, 16 * nt, dl);
  }
  __syncthreads();
  GDR_POISON(Pt, Ly::F);  // Pt and the float32 L^{-1} are no longer read
  GDR_POISON(Li, Ly::F);
  {  // dbeta from L = I + diag(beta) A: row sums (dL is zero on and above the diagonal); eight
     // adjacent lanes per row, eight consecutive columns each (vector reads), summed with DPP
    static_assert(NT == 8 * CH, "eight lanes per row");
    const int t = threadIdx.x >> 3, s0 = (threadIdx.x & 7) * 8;
    const float4 l0 = *reinterpret_cast<const float4*>(dTs + t * LF + s0);
    const float4 l1 = *reinterpret_cast<const float4*>(dTs + t * LF + s0 + 4);
    const float4 a0 = *reinterpret_cast<const float4*>(As + t * LF + s0);
    const float4 a1 = *reinterpret_cast<const float4*>(As + t * LF + s0 + 4);
    float a = l0.x * a0.x + l0.y * a0.y + l0.z * a0.z + l0.w * a0.w + l1.x * a1.x + l1.y * a1.y + l1.z * a1.z +
              l1.w * a1.w;
    a = group_sum_dpp<8>(a);
    if ((threadIdx.x & 7) == 0) pdb[t] = a;
  }

  // ================= phase 3: Gram slots and the decay gradient
  E* Qs = reinterpret_cast<E*>(smem + Ly::oQ);
  E* Ats = reinterpret_cast<E*>(smem + Ly::oAt);
  E* Mts = reinterpret_cast<E*>(smem + Ly::oMt);
  float* Pair = reinterpret_cast<float*>(smem + Ly::oPair);
  if constexpr (QKN) scale_rows(pQ, rnq);
  pQ.store(Qs, LD);
  // Each thread handles the (t, s) entries of M it holds in registers.
  {  // VE consecutive columns per thread: vector LDS reads and writes
    using RM = RegTile<E, CH, CH, NT>;
    constexpr int VE = RM::VE;
    static_assert(VE % 4 == 0, "four float columns per vector");
#pragma unroll
    for (int it = 0; it < RM::IT; ++it) {
      if (RM::TOTAL % NT == 0 || threadIdx.x + it * NT < RM::TOTAL) {
        const int t = pM.row(it), s0 = pM.col(it);
        const float gt = gs[t], bt = bs[t];
        float dTv[VE], Av[VE], gv[VE];
#pragma unroll
        for (int e = 0; e < VE; e += 4) {
          const float4 x = *reinterpret_cast<const float4*>(dTs + t * LF + s0 + e);
          dTv[e] = x.x; dTv[e + 1] = x.y; dTv[e + 2] = x.z; dTv[e + 3] = x.w;
          const float4 y = *reinterpret_cast<const float4*>(gs + s0 + e);
          gv[e] = y.x; gv[e + 1] = y.y; gv[e + 2] = y.z; gv[e + 3] = y.w;
          if constexpr (GATED) {
            const float4 a = *reinterpret_cast<const float4*>(As + t * LF + s0 + e);
            Av[e] = a.x; Av[e + 1] = a.y; Av[e + 2] = a.z; Av[e + 3] = a.w;
          }
        }
        typename RM::V mv = *reinterpret_cast<const typename RM::V*>(dMs + t * LDR + s0), av, tv;
        const E* me = reinterpret_cast<const E*>(&mv);
        E* ae = reinterpret_cast<E*>(&av);
        E* te = reinterpret_cast<E*>(&tv);
        float pr[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int s = s0 + e;
          float dec = 0.f;
          if (s <= t) {
            dec = 1.f;
            if constexpr (GATED) dec = __expf(gt - gv[e]);
          }
          const float dA = (s < t) ? bt * dTv[e] : 0.f;
          const float dM = (s <= t) ? (float)me[e] : 0.f;
          ae[e] = (E)(dA * dec);
          te[e] = (E)(dM * dec);
          pr[e] = 0.f;
          if constexpr (GATED) pr[e] = (s < t) ? dA * Av[e] + dM * (float)pM.elem(it, e) : 0.f;
        }
        *reinterpret_cast<typename RM::V*>(Ats + t * LDR + s0) = av;
        *reinterpret_cast<typename RM::V*>(Mts + t * LDR + s0) = tv;
        if constexpr (GATED) {
#pragma unroll
          for (int e = 0; e < VE; e += 4)
            *reinterpret_cast<float4*>(Pair + t * LF + s0 + e) = make_float4(pr[e], pr[e + 1], pr[e + 2], pr[e + 3]);
        }
      }
    }
  }
  __syncthreads();
  GDR_POISON(As, Ly::F);  // A, dT (now dL) and dM are no longer read
  GDR_POISON(dTs, Ly::F);
  GDR_POISON(dMs, Ly::SQ);
  if (w < 4) {  // the row's Qhat . dQhat (state term), four consecutive columns per lane
    float part = 0.f;
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const f32x4 qv = get4(Qs + tr * LD + 16 * nt + 4 * lgrp());
      part += qv[0] * acc1[nt][0] + qv[1] * acc1[nt][1] + qv[2] * acc1[nt][2] + qv[3] * acc1[nt][3];
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rq[w][tr] = part;
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = mma_k<E, CH>(acc1[nt], colk(Ks, LD), 16 * nt, rowk(Mts, LDR), 16 * wm);
    if constexpr (QKN) {  // dq~ is complete: dq = (dq~ - q~ (q~ . dq~)) / ||q|| at once, this wave
      // holding every column of rows tr.  Done after the remaining products instead, it kept
      // acc1 live across them and the D = 128 kernels spilled some 600 registers.
      float dot = 0.f;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const f32x4 qv = get4(Qs + tr * LD + 16 * nt + 4 * lgrp());
        dot += qv[0] * acc1[nt][0] + qv[1] * acc1[nt][1] + qv[2] * acc1[nt][2] + qv[3] * acc1[nt][3];
      }
      dot = sum_rows4(dot);
      const float rn = invq[tr];
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = (acc1[nt] - dot * get4(Qs + tr * LD + 16 * nt + 4 * lgrp())) * rn;
    }
  }
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int nt = wn * NQ + qq;
    dka[qq] = mma_k<E, CH>(dka[qq], colk(Ks, LD), 16 * nt, rowk(Ats, LDR), 16 * wm);
    dka[qq] = mma_k<E, CH>(dka[qq], colk(Ks, LD), 16 * nt, colk(Ats, LDR), 16 * wm);
    dka[qq] = mma_k<E, CH>(dka[qq], colk(Qs, LD), 16 * nt, colk(Mts, LDR), 16 * wm);
  }
  if constexpr (QKN) {  // dk~ is complete: k~ . dk~ over this wave's columns of rows tr (a row's
    // columns are split over waves w and w ^ 4), summed after the next barrier
    float part = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const f32x4 kv = get4(Ks + tr * LD + 16 * (wn * NQ + qq) + 4 * lgrp());
      part += kv[0] * dka[qq][0] + kv[1] * dka[qq][1] + kv[2] * dka[qq][2] + kv[3] * dka[qq][3];
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rkn[w][tr] = part;
  }
  if constexpr (GATED) {  // prefix sums along each row of the pair terms: lanes over columns
#pragma unroll
    for (int i = 0; i < CH / (NT / 64); ++i) {  // rows w, w + 8, ...: independent, interleaved
      float* row = Pair + (w + i * (NT / 64)) * LF;
      row[lane_id()] = wave_incl_scan(row[lane_id()]);
    }
  }
  __syncthreads();
  GDR_POISON(smem + Ly::odR, 2 * Ly::SQ);  // At, Mt and Q are no longer read
  GDR_POISON(Qs, Ly::TK);
  if constexpr (QKN) {  // dk w.r.t. the raw rows: dk = (dk~ - k~ (k~ . dk~)) / ||k|| (dq was done above)
    const float dot = rkn[wm][tr] + rkn[wm + 4][tr];
    const float rn = invk[tr];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq)
      dka[qq] = (dka[qq] - dot * get4(Ks + tr * LD + 16 * (wn * NQ + qq) + 4 * lgrp())) * rn;
  }
  if constexpr (GATED) {  // rectangle sums: sum over u >= t of the prefix at column t-1
    const int t = threadIdx.x & (CH - 1), pt = threadIdx.x >> 6;
    float a = 0.f;
    if (t > 0) {
#pragma unroll
      for (int i = 0; i < CH / (NT / CH); ++i) {
        const int uu = pt + i * (NT / CH);
        a += (uu >= t) ? Pair[uu * LF + t - 1] : 0.f;
      }
    }
    part8[pt][t] = a;
  }
  __syncthreads();
  GDR_POISON(smem + Ly::oPair, Ly::F);  // the pair terms are no longer read
  // outputs: dq, dk through LDS (the dR/dX regions are free now)
  E* sq = reinterpret_cast<E*>(smem + Ly::odR);
  E* sk = reinterpret_cast<E*>(smem + Ly::odX);
  if (w < 4) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) store4_t(sq, LD, 16 * nt, 16 * wm, acc1[nt]);
  }
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) store4_t(sk, LD, 16 * (wn * NQ + qq), 16 * wm, dka[qq]);
  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    if constexpr (GATED) {
      float rect = 0.f;  // sum over u >= t of sum_{s < t} pair(u, s)
#pragma unroll
      for (int i = 0; i < NT / CH; ++i) rect += part8[i][t];
      // suffix over u >= t of the rows' Qhat.dQhat + Khat.dKhat (reversed inclusive scan)
      const int tq = CH - 1 - t;
      const float xr = rq[tq >> 4][tq] + rkh[tq >> 4][tq] + rkh[(tq >> 4) + 4][tq];
      const float suf_r = wave_incl_scan(xr);
      const float suf = __shfl(suf_r, CH - 1 - t, 64);
      // prefix over s < t of Kbar.dKbar (exclusive scan)
      const float xb = rkb[t >> 4][t] + rkb[(t >> 4) + 4][t];
      const float inc = wave_incl_scan(xb);
      float pre = __shfl_up(inc, 1, 64);
      if (t == 0) pre = 0.f;
      float g4 = 0.f;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) g4 += red[i];
      const float dla = rect + suf + pre + __expf(gn) * g4;
      if (t < n) {
        if constexpr (LOG) dalpha[tk + t] = (E)(-dla * gate_sigmoid((float)araw));
        else dalpha[tk + t] = (E)(dla / (float)araw);
      }
    }
    float db = pdb[t];
#pragma unroll
    for (int i = 0; i < NT / CH; ++i) db += part8c[i][t];
    if constexpr (RES) {
      if (t < n) {
        const float bi = 1.f / (float)braw;
        db -= rdr[t] * bi * bi;
      }
    }
    if constexpr (LOG) db *= bs[t] * (1.f - bs[t]);
    if (t < n) dbeta[tk + t] = (E)db;
  }
  __syncthreads();
  s2g_rows<E, CH, D, NT>(dq + tk * D, D, sq, LD, n);
  s2g_rows<E, CH, D, NT>(dk + tk * D, D, sk, LD, n);
}

// ---------------------------------------------------------------------------------------
// The beta gradient when the residual r = R / beta was an output (its gradient dr given).
// ---------------------------------------------------------------------------------------
// Fed with dR + dr / beta, the chunk kernel's beta gradient holds two terms of order
// |dr| |r| / beta that cancel exactly (the dr / beta in dR against the -dr.R / beta^2 of
// r = R / beta), and with bfloat16 operands their rounding is larger than the result at small
// beta.  The sum is linear, so the beta gradient is instead formed as
//   dbeta = F(dR_o) + G,
// where dR_o = M^T dO + Kbar dW^T is dR without the residual's term and F is the chunk
// kernel's beta gradient for a given dR,
//   dT = dR_o Y^T (Y = V - Khat W0^T = r + A R, since R = L^{-1} diag(beta) Y),
//   F_s = sum_t dT_ts Linv_ts + sum_s' dL_ss' A_ss',  dL = -strictlower(L^-T dT diag(beta) L^-T),
// and G is the residual's own term, from r = Lt^{-1} Y with Lt = I + A diag(beta):
//   dY = Lt^-T dr = diag(beta) L^-T (dr / beta),  G_s = -r_s . (A^T dY)_s.
// Neither part carries a term of order 1 / beta that another cancels.  The chunk kernel's
// beta gradient is overwritten.  One workgroup of 512 threads per (chunk, head).
// OWN_A (delta family): A is formed from K and the log decays as the forward formed it (the
// forward keeps no copy); otherwise (Kimi Delta Attention) it is read from the forward's cache.
template <typename E, int D, bool OWN_A, bool QKN>
__global__ __launch_bounds__(512) void k_bwd_res_dbeta(Geo geo, const E* __restrict__ Rg, const E* __restrict__ dRog,
                                                       const E* __restrict__ drin, const E* __restrict__ beta,
                                                       const float* __restrict__ Ag, const E* __restrict__ k,
                                                       const float* __restrict__ Gg, const float* __restrict__ Lig,
                                                       E* __restrict__ dbeta, const float* __restrict__ Rng) {
  GDR_POISON_ALL();
  constexpr int NT = 512, LD = D + pad16<E>(), LF = CH + 4, NW = NT / 64;
  constexpr int NH = D / 32;  // column tiles of a 64 x D product per wave (two waves per row block)
  constexpr int TE = CH * LD, TF = CH * LF;
  __shared__ __align__(16) E Rs[TE], dRos[TE], Ds[TE], Ys[TE];  // Ys later holds dY
  __shared__ __align__(16) float As[TF], Lis[TF], dTs[TF], Pts[TF];
  __shared__ float bs[CH], binv[CH], colp[NW][CH], rowp[CH], gz[2][CH], gs[OWN_A ? CH : 1];
  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int n = cp.n, wm = wave_id() & 3, wn = wave_id() >> 2;  // row block, column half

  const uint32_t braw = threadIdx.x < CH ? load_gate_raw(beta + tk, n, threadIdx.x) : 0u;
  float graw = 0.f;
  if constexpr (OWN_A) {
    if (threadIdx.x < CH) graw = Gg[u * CH + threadIdx.x];
  }
  {
    RegTile<E, CH, D, NT> rR, rO, rd, rk;
    RegTile<float, CH, CH, NT> rA, rL;
    float rnk[decltype(rk)::IT];  // QKN: 1 / ||k|| of the rows of rk this thread holds
    if constexpr (OWN_A) {
      if constexpr (QKN) load_row_factors(rk, Rng + u * 2 * CH + CH, rnk);  // before the tiles
      rk.load(k + tk * D, D, n);
    } else {
      rA.load(Ag + u * CH * CH, CH, CH);
    }
    rR.load(Rg + u * CH * D, D, CH);
    rO.load(dRog + u * CH * D, D, CH);
    rL.load(Lig + u * CH * CH, CH, CH);
    rd.load(drin + tk * D, D, n);
    if constexpr (OWN_A) {  // K (scaled to unit length as the forward scaled it), in the region Y takes later
      if constexpr (QKN) scale_rows(rk, rnk);
      rk.store(Ys, LD);
    }
    rR.store(Rs, LD);
    rO.store(dRos, LD);
    if (threadIdx.x < CH) {
      const float b = gate_from_raw<E>(braw);  // 0 past the end
      bs[threadIdx.x] = b;
      binv[threadIdx.x] = threadIdx.x < n ? 1.f / b : 0.f;
      if constexpr (OWN_A) gs[threadIdx.x] = graw;
    }
    if constexpr (!OWN_A) rA.store(As, LF);
    rL.store(Lis, LF);
    __syncthreads();
    if constexpr (OWN_A) {  // A = strictlower(K K^T) e^{g_t - g_s}, the forward's products
      const int w = wave_id();
#pragma unroll
      for (int job_r = 0; job_r < ((10) + (NT / 64) - 1) / (NT / 64); ++job_r) {
        const int job = w + job_r * (NT / 64);
        if (job >= 10) break;
        int mt, nt;
        tri_tile(job, mt, nt);
        const f32x4 acc = mma_k<E, D>(zero4(), rowk(Ys, LD), 16 * nt, rowk(Ys, LD), 16 * mt);
        const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
        float val[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sc = s0 + r;
          val[r] = sc < t ? acc[r] * __expf(gs[t] - gs[sc]) : 0.f;
        }
        *reinterpret_cast<float4*>(As + t * LF + s0) = make_float4(val[0], val[1], val[2], val[3]);
      }
#pragma unroll
      for (int idx_r = 0; idx_r < ((CH * CH / 4) + NT - 1) / NT; ++idx_r) {
        const int idx = (int)threadIdx.x + idx_r * NT;
        if (idx >= CH * CH / 4) break;
        const int t = idx >> 4, s0 = (idx & 15) * 4;
        if ((s0 >> 4) > (t >> 4)) *reinterpret_cast<float4*>(As + t * LF + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int it = 0; it < decltype(rd)::IT; ++it) {  // dr / beta, zero past the end
      const int r = rd.row(it), c = rd.col(it);
      const float bi = binv[r];
#pragma unroll
      for (int x = 0; x < decltype(rd)::VE; ++x) Ds[r * LD + c + x] = (E)((float)rd.elem(it, x) * bi);
    }
  }
  __syncthreads();  // A complete (and, with OWN_A, K read) before Y overwrites K
  // Y = R / beta + A R; wave (wm, wn) forms rows 16 wm .. 16 wm + 15, column tiles of half wn
#pragma unroll
  for (int q = 0; q < NH; ++q) {
    const int nt = wn * NH + q;
    f32x4 y = mma_k<E, CH>(zero4(), rowk(As, LF), 16 * wm, colk(Rs, LD), 16 * nt);
    const int j = acc_col(16 * nt);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = acc_row(16 * wm, r);
      y[r] += (float)Rs[t * LD + j] * binv[t];
    }
    store4_n(Ys, LD, 16 * wm, 16 * nt, y);
  }
  __syncthreads();
  // dT = dR_o Y^T on and below the diagonal
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * wn + q;
    const f32x4 a = mma_k<E, D>(zero4(), rowk(dRos, LD), 16 * wm, rowk(Ys, LD), 16 * nt);
    const int sc = acc_col(16 * nt);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = acc_row(16 * wm, r);
      dTs[t * LF + sc] = sc <= t ? a[r] : 0.f;
    }
  }
  __syncthreads();
  {  // F from T = Linv diag(beta): column sums, eight threads per column
    const int sc = threadIdx.x & (CH - 1), pt = threadIdx.x >> 6;
    float a = 0.f;
#pragma unroll
    for (int t = pt, t_r = 0; t_r < CH / (NW); ++t_r, t += NW) a += dTs[t * LF + sc] * Lis[t * LF + sc];
    colp[pt][sc] = a;
  }
  // Pt = (dT diag(beta)) Linv^T, stored transposed
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * wn + q;
    const f32x4 acc = mma_k<E, CH>(zero4(), RowKScaled{dTs, LF, bs}, 16 * wm, rowk(Lis, LF), 16 * nt);
    store4_t(Pts, LF, 16 * wm, 16 * nt, acc);
  }
  __syncthreads();
  // dL = -strictlower(Linv^T Pt) over dT
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * wn + q;
    const f32x4 acc = mma_k<E, CH>(zero4(), colk(Lis, LF), 16 * wm, rowk(Pts, LF), 16 * nt);
    f32x4 dl;
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[r] = (acc_col(16 * nt) < acc_row(16 * wm, r)) ? -acc[r] : 0.f;
    store4_n(dTs, LF, 16 * wm, 16 * nt, dl);
  }
  // dY = diag(beta) Linv^T (dr / beta), over Y (free once dT is formed)
#pragma unroll
  for (int q = 0; q < NH; ++q) {
    const int nt = wn * NH + q;
    f32x4 y = mma_k<E, CH>(zero4(), colk(Lis, LF), 16 * wm, colk(Ds, LD), 16 * nt);
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] *= bs[acc_row(16 * wm, r)];
    store4_n(Ys, LD, 16 * wm, 16 * nt, y);
  }
  __syncthreads();
  if (threadIdx.x < CH) {  // F from L = I + diag(beta) A: row sums
    const int t = threadIdx.x;
    float a = 0.f;
    for (int sc = 0; sc < t; ++sc) a += dTs[t * LF + sc] * As[t * LF + sc];
    rowp[t] = a;
  }
  {  // G_s = -sum_j r_sj (A^T dY)_sj: rows 16 wm .. 16 wm + 15, columns of half wn
    f32x4 g = zero4();
#pragma unroll
    for (int q = 0; q < NH; ++q) {
      const int nt = wn * NH + q;
      const f32x4 z = mma_k<E, CH>(zero4(), colk(As, LF), 16 * wm, colk(Ys, LD), 16 * nt);
      const int j = acc_col(16 * nt);
#pragma unroll
      for (int r = 0; r < 4; ++r) g[r] += (float)Rs[acc_row(16 * wm, r) * LD + j] * z[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) g[r] += __shfl_xor(g[r], off, 64);
    }
    if (lrow() == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sr = acc_row(16 * wm, r);
        gz[wn][sr] = -g[r] * binv[sr];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < n) {
    const int t = threadIdx.x;
    float db = rowp[t] + gz[0][t] + gz[1][t];
#pragma unroll
    for (int i = 0; i < NW; ++i) db += colp[i][t];
    dbeta[tk + t] = (E)db;
  }
}

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
template <typename E, int D, int VAR>
static hipError_t bwd_impl(const Plan& p, const gdr_inputs& in, const void* dO, const void* dr, const float* dht,
                           const gdr_grads& gr, hipStream_t st) {
  const Geo& g = p.geo;
  constexpr bool KDA = VAR == VAR_KDA;
  constexpr bool PCH = KDA || VAR == VAR_GLA;  // decay per key channel: per-unit operands
  const E* qin = PCH ? (const E*)p.Qh : (const E*)in.q;
  const E* kin = PCH ? (const E*)p.Kb : (const E*)in.k;
  const float* gin = PCH ? p.Gn : p.G;
  // residual gradient: delta family and Kimi Delta Attention (whose residual has the same form)
  constexpr bool RES_OK = VAR == VAR_DELTANET || VAR == VAR_GATED || KDA;
  const E* drp = RES_OK ? (const E*)dr : nullptr;
  // The beta gradient of a residual output is formed apart (k_bwd_res_dbeta) from dR without the
  // residual's term, which the scan then also records, over U (not read backward): with
  // bfloat16 I/O for the delta family, whose chunk kernel otherwise adds the direct term itself,
  // and always for Kimi Delta Attention, whose backward stages take no residual.
  E* dro = (RES_OK && drp && (KDA || std::is_same<E, bf16>::value)) ? (E*)p.Ub : nullptr;
  auto launch = [&](auto kern, int bv, const ScanSeg& sg, const float* dhtp, float* dh0p, int nv_mult, const E* d) {
    const int ny = (sg.mode == 1 || sg.mode == 2) ? sg.max_seg : 1;  // mode 3: one segment per sequence
    hipLaunchKernelGGL(kern, dim3(scan_grid(g, nv_mult * D / bv), ny), dim3(256), 0, st, g, sg,
                       qin, kin, (const E*)dO, (const E*)p.X, (const E*)p.M, gin, dhtp, (E*)p.dHs, (E*)p.dR, dh0p,
                       (const E*)in.beta, (const E*)in.erase, d, d ? dro : nullptr, (const float*)p.Rn);
  };
  constexpr bool QOK = VAR == VAR_DELTANET || VAR == VAR_GATED;  // fused q/k normalisation
  auto scan_q = [&](auto qkn, const ScanSeg& sg, const float* dhtp, float* dh0p, int nv_mult) {
    constexpr bool Q = decltype(qkn)::value;
    if (p.bv == 16) {
      if constexpr (RES_OK) {
        if (drp) return launch(k_bwd_scan<E, D, 16, VAR, true, Q>, 16, sg, dhtp, dh0p, nv_mult, drp);
      }
      launch(k_bwd_scan<E, D, 16, VAR, false, Q>, 16, sg, dhtp, dh0p, nv_mult, nullptr);
    } else {
      if constexpr (RES_OK) {
        if (drp) return launch(k_bwd_scan<E, D, 32, VAR, true, Q>, 32, sg, dhtp, dh0p, nv_mult, drp);
      }
      launch(k_bwd_scan<E, D, 32, VAR, false, Q>, 32, sg, dhtp, dh0p, nv_mult, nullptr);
    }
  };
  auto scan = [&](const ScanSeg& sg, const float* dhtp, float* dh0p, int nv_mult) {
    if constexpr (!PCH) {
      if (p.qkn) return scan_q(std::true_type{}, sg, dhtp, dh0p, nv_mult);
    }
    scan_q(std::false_type{}, sg, dhtp, dh0p, nv_mult);
  };
  // the chunk-parallel gradients of the delta family, over every chunk (grid (chunks, H)) or,
  // with lseg > 0, over part `part` of every sequence (grid (lseg, H, sequences))
  auto chunk_grads = [&](hipStream_t cs, int part, int lseg) {
    const dim3 grid = lseg > 0 ? dim3(lseg, g.H, g.nseq) : dim3(g.total_chunks, g.H);
    auto chunk = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(512), 0, cs, g, qin, kin,
                         (const E*)in.v, (const E*)in.beta, (const E*)in.alpha, (const E*)dO, (const E*)p.M,
                         (const float*)p.G, (const E*)p.Hs, (const E*)p.R, (const E*)p.dHs, (const E*)p.dR,
                         p.Li, (E*)gr.dq, (E*)gr.dk, (E*)gr.dv, (E*)gr.dbeta, (E*)gr.dalpha, drp,
                         (const float*)p.Rn, part, lseg);
    };
    if constexpr (!PCH && VAR != VAR_GDN2 && VAR != VAR_GDN2L) {
      if (p.qkn) {
        if (drp) chunk(k_bwd_chunk<E, D, VAR, true, false, true>);
        else if (p.gates) chunk(k_bwd_chunk<E, D, VAR, false, true, true>);
        else chunk(k_bwd_chunk<E, D, VAR, false, false, true>);
      } else {
        if (drp) chunk(k_bwd_chunk<E, D, VAR, true, false, false>);
        else if (p.gates) chunk(k_bwd_chunk<E, D, VAR, false, true, false>);
        else chunk(k_bwd_chunk<E, D, VAR, false, false, false>);
      }
    }
  };
  // Time-split backward (delta family, unsegmented reverse scan, a side stream given): the
  // reverse scan runs part by part (ScanSeg mode 3) on the caller's stream, and each finished
  // part's chunk gradients run on the side stream while the next part scans, on the CUs the
  // scan's few value tiles leave idle.  The side stream is joined back into the caller's
  // stream before anything else is enqueued, also after an error.
  constexpr bool DELTA = VAR == VAR_DELTANET || VAR == VAR_GATED;
  const bool tsplit = DELTA && p.ts_lseg > 0 && p.ts_side && p.lseg_b == 0 && g.total_chunks > 0;
  if (tsplit) {
    hipError_t e = hipSuccess;
    bool forked = false;
    for (int part = 0; part < p.ts_parts && e == hipSuccess; ++part) {
      {
        TraceScope ts_("bwd_scan", st);
        scan(ScanSeg{3, p.ts_lseg, p.ts_parts, p.seg_maps, nullptr, part}, dht, gr.dh0, 1);
      }
      if ((e = hipGetLastError()) != hipSuccess) break;
      if ((e = hipEventRecord(p.ts_fork, st)) != hipSuccess) break;
      if ((e = hipStreamWaitEvent(p.ts_side, p.ts_fork, 0)) != hipSuccess) break;
      forked = true;
      TraceScope ts_("bwd_chunk", p.ts_side);
      chunk_grads(p.ts_side, part, p.ts_lseg);
      e = hipGetLastError();
    }
    if (forked) {
      hipError_t j = hipEventRecord(p.ts_join, p.ts_side);
      if (j == hipSuccess) j = hipStreamWaitEvent(st, p.ts_join, 0);
      if (j != hipSuccess) {
        (void)hipStreamSynchronize(p.ts_side);  // the ordering could not be expressed on the stream
        if (e == hipSuccess) e = j;
      }
    }
    if (e != hipSuccess) return e;
  } else if (p.lseg_b == 0) {
    TraceScope ts_("bwd_scan", st);
    scan(ScanSeg{0, 0, 1, nullptr, nullptr, 0}, dht, gr.dh0, 1);
  } else {
    {
      TraceScope ts_("bwd_scan_maps", st);
      scan(ScanSeg{1, p.lseg_b, p.max_seg_b, p.seg_maps, nullptr, 0}, nullptr, nullptr, 2);
    }
    const hipError_t e = launch_seg_combine(p, ScanSeg{0, p.lseg_b, p.max_seg_b, p.seg_maps, nullptr, 0}, dht, true, st);
    if (e != hipSuccess) return e;
    TraceScope ts_("bwd_scan", st);
    scan(ScanSeg{2, p.lseg_b, p.max_seg_b, nullptr, p.seg_starts, 0}, nullptr, gr.dh0, 1);
  }
  if (g.total_chunks > 0) {
    if constexpr (VAR == VAR_GDN2 || VAR == VAR_GDN2L) {
      return launch_bwd_gdn2<E, D>(p, in, dO, gr, st);
    } else if constexpr (PCH) {
      const hipError_t e = launch_bwd_kda<E, D>(p, in, dO, gr, st);
      if (e != hipSuccess) return e;
    } else if (!tsplit) {  // (time-split: done above)
      TraceScope ts_("bwd_chunk", st);
      chunk_grads(st, 0, 0);
    }
    if constexpr (RES_OK) {
      if (dro) {
        TraceScope ts_("bwd_res_dbeta", st);
        auto res = [&](auto kern) {
          hipLaunchKernelGGL(kern, dim3(g.total_chunks, g.H), dim3(512), 0, st, g, (const E*)p.R,
                             (const E*)dro, drp, (const E*)in.beta, (const float*)p.A1, kin, gin,
                             (const float*)p.Li, (E*)gr.dbeta, (const float*)p.Rn);
        };
        if constexpr (QOK) {
          if (p.qkn) res(k_bwd_res_dbeta<E, D, true, true>);
          else res(k_bwd_res_dbeta<E, D, true, false>);
        } else {
          res(k_bwd_res_dbeta<E, D, false, false>);
        }
      }
    }
  }
  return hipGetLastError();
}

hipError_t run_backward(const Plan& p, const gdr_inputs& in, const void* dO, const void* dr, const float* dht,
                        const gdr_grads& gr, hipStream_t st) {
  const bool bf = p.dtype == GDR_BF16;
#define GDR_BWD_CASE(V)                                                                  \
  if (bf && p.D == 128) return bwd_impl<bf16, 128, V>(p, in, dO, dr, dht, gr, st);       \
  if (bf && p.D == 64) return bwd_impl<bf16, 64, V>(p, in, dO, dr, dht, gr, st);         \
  if (!bf && p.D == 64) return bwd_impl<float, 64, V>(p, in, dO, dr, dht, gr, st);       \
  break;
  switch (p.variant) {
    case GDR_DELTANET: GDR_BWD_CASE(VAR_DELTANET)
    case GDR_GATED: GDR_BWD_CASE(VAR_GATED)
    case GDR_KDA: GDR_BWD_CASE(VAR_KDA)
    case GDR_GLA: GDR_BWD_CASE(VAR_GLA)
    case GDR_GDN2:
      if (p.gates) { GDR_BWD_CASE(VAR_GDN2L) }
      GDR_BWD_CASE(VAR_GDN2)
    default: break;
  }
#undef GDR_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdr
