// Forward kernels of the chunked delta-rule operator (Delta family: DeltaNet, Gated DeltaNet).
//
// Chunk form of the token recurrence (per chunk of n <= 64 tokens starting from memory W0,
// g_t = sum_{u<=t} log alpha_u inside the chunk, E_ts = exp(g_t - g_s) for s <= t):
//   A_ts = (k_t . k_s) E_ts (s < t),  M_ts = (q_t . k_s) E_ts (s <= t)
//   L = I + diag(beta) A,  T = L^{-1} diag(beta)
//   X = T (e^g * K),  U = T V                      (WY/UT factors of prod (I - beta k k^T))
//   R = U - X W0^T                                  (row t: beta_t times the residual r_t)
//   O = scale * ((e^g * Q) W0^T + M R)
//   W_next = e^{g_n} W0 + R^T (e^{g_n - g} * K)
// Two launches: a chunk-parallel prep (A, M, L^{-1}, X, U) and a sequential scan over the
// chunks of each (sequence, head, value-row tile) that carries W in float32 registers, records
// W0 and R per chunk and writes the tile's output columns (segmented scans add a map pass and
// a combine, see seg.hip).
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

// ---------------------------------------------------------------------------------------
// Prep: per (head, chunk) -- g, M, L^{-1}, X, U.
// ---------------------------------------------------------------------------------------
// LOG: beta and alpha are logits (beta = sigmoid(x), log alpha = -softplus(x)).
// QKN: q and k are scaled to unit length per token as they are loaded (normalize_rows), and
// 1/||q||, 1/||k|| are kept per unit in Rno (zero for a zero row and past the sequence's end);
// the later kernels read the raw rows and apply those factors themselves.
template <typename E, int D, int VAR, bool LOG, bool QKN>
__global__ __launch_bounds__(256) void k_fwd_prep(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                  const E* __restrict__ v, const E* __restrict__ beta,
                                                  const E* __restrict__ alpha, E* __restrict__ Xo,
                                                  E* __restrict__ Uo, E* __restrict__ Mo, float* __restrict__ Go,
                                                  float* __restrict__ Lio, float* __restrict__ Rno) {
  GDR_POISON_ALL();
  constexpr int NT = 256, LD = D + pad16<E>(), LDT = CH + pad16<E>(), LF = CH + 4;
  // Three 64-row buffers (about 52 KiB, so three workgroups share a CU):
  static_assert(CH * LD * (int)sizeof(E) >= 4 * 256 * 4, "the Q/V buffer doubles as the solve's scratch");
  static_assert(LDT * (int)sizeof(E) <= LF * 4, "T fits the buffer of L");
  __shared__ __align__(16) E Ks[CH * LD];     // K, then e^g * K, then X
  __shared__ __align__(16) E QV[CH * LD];     // Q, then the solve's scratch, then V, then U
  __shared__ __align__(16) float Ls[CH * LF];  // L, then L^{-1} (solved in place), then T = L^{-1} diag(beta)
  E* Ts = reinterpret_cast<E*>(Ls);
  __shared__ __align__(16) float gs[CH], bs[CH];

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id();

  // The gates are loaded before the tiles (plain loads of a valid token) and used after the
  // K and Q stores: their waits then cover nothing the stores did not already need, where
  // loaded after the tiles they would also wait for V.
  E braw = E(0.f), araw = E(1.f);
  if (threadIdx.x < CH) {
    const int t = min((int)threadIdx.x, cp.n - 1);
    braw = beta[tk + t];
    if constexpr (VAR == VAR_GATED) araw = alpha[tk + t];
  }
  RegTile<E, CH, D, NT> rk, rq, rv;
  rk.load(k + tk * D, D, cp.n);
  rq.load(q + tk * D, D, cp.n);
  rv.load(v + tk * D, D, cp.n);
  if constexpr (QKN) {
    normalize_rows(rq, Rno + u * 2 * CH);
    normalize_rows(rk, Rno + u * 2 * CH + CH);
  }
  rk.store(Ks, LD);
  rq.store(QV, LD);
  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    const bool ok = t < cp.n;
    float la = 0.f;
    if constexpr (LOG) {
      bs[t] = ok ? gate_sigmoid((float)braw) : 0.f;
      if constexpr (VAR == VAR_GATED) la = ok ? gate_neg_softplus((float)araw) : 0.f;
    } else {
      bs[t] = ok ? (float)braw : 0.f;
      if constexpr (VAR == VAR_GATED) la = ok ? logf((float)araw) : 0.f;
    }
    const float g = wave_incl_scan(la);
    gs[t] = g;
    Go[u * CH + t] = g;
  }
  __syncthreads();

  // Gram tiles: jobs 0..9 -> A (strict lower, times beta_t, into Ls), 10..19 -> M (lower).
  // Formed transposed, so each lane holds four consecutive columns s of one row t and writes
  // them with one vector store.
  // five jobs per wave, unrolled so that one job's operand reads overlap another's products
#pragma unroll
  for (int jr = 0; jr < 5; ++jr) {
    const int job = w + 4 * jr;
    const bool isM = jr >= 3 || (jr == 2 && w >= 2);  // job >= 10
    int mt, nt;
    tri_tile(isM ? job - 10 : job, mt, nt);
    const f32x4 acc = mma_k<E, D>(zero4(), rowk(Ks, LD), 16 * nt, rowk(isM ? QV : Ks, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    float val[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + r;
      const bool keep = isM ? (s <= t) : (s < t);
      float dec = 1.f;
      if constexpr (VAR == VAR_GATED) dec = __expf(gs[t] - gs[s]);
      val[r] = keep ? acc[r] * dec : 0.f;
    }
    if (isM) {
      if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<bf16x4*>(Mo + (u * CH + t) * CH + s0) = bf16x4{(E)val[0], (E)val[1], (E)val[2], (E)val[3]};
      } else {
        *reinterpret_cast<float4*>(Mo + (u * CH + t) * CH + s0) = make_float4(val[0], val[1], val[2], val[3]);
      }
    } else {
      const float bt = bs[t];
      *reinterpret_cast<float4*>(Ls + t * LF + s0) = make_float4(bt * val[0], bt * val[1], bt * val[2], bt * val[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < CH * CH / 4 / NT; ++i) {  // tiles above the diagonal
    const int idx = threadIdx.x + i * NT, t = idx >> 4, s0 = (idx & 15) * 4;
    if ((s0 >> 4) > (t >> 4)) {
      if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<bf16x4*>(Mo + (u * CH + t) * CH + s0) = bf16x4{(E)0.f, (E)0.f, (E)0.f, (E)0.f};
      } else {
        *reinterpret_cast<float4*>(Mo + (u * CH + t) * CH + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  __syncthreads();
  GDR_POISON(QV, (int)sizeof(QV));  // Q is no longer read
  solve_unit_lower64<NT>(Ls, LF, Ls, LF, reinterpret_cast<float*>(QV));
  GDR_POISON(QV, (int)sizeof(QV));  // nor the solve's scratch
  rv.store(QV, LD);

  // T = L^{-1} diag(beta), four columns at a time: L^{-1} is read into registers (and written
  // out for the backward) before T overwrites it in the same buffer
  constexpr int TI = CH * CH / 4 / NT;
  float tv[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int idx = threadIdx.x + i * NT, t = idx >> 4, s0 = (idx & 15) * 4;
    const float4 l = *reinterpret_cast<const float4*>(Ls + t * LF + s0);
    *reinterpret_cast<float4*>(Lio + u * CH * CH + t * CH + s0) = l;  // L^{-1} for the backward
    const float4 bb = *reinterpret_cast<const float4*>(bs + s0);
    const float lv[4] = {l.x * bb.x, l.y * bb.y, l.z * bb.z, l.w * bb.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) tv[i][r] = s0 + r <= t ? lv[r] : 0.f;
  }
  __syncthreads();
  GDR_POISON(Ls, (int)sizeof(Ls));  // L^{-1} is held in registers
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int idx = threadIdx.x + i * NT, t = idx >> 4, s0 = (idx & 15) * 4;
    if constexpr (sizeof(E) == 2) {
      *reinterpret_cast<bf16x4*>(Ts + t * LDT + s0) = bf16x4{(E)tv[i][0], (E)tv[i][1], (E)tv[i][2], (E)tv[i][3]};
    } else {
      *reinterpret_cast<float4*>(Ts + t * LDT + s0) = make_float4(tv[i][0], tv[i][1], tv[i][2], tv[i][3]);
    }
  }
  if constexpr (VAR == VAR_GATED) {  // Khat = e^g K in place, 16 bytes at a time
    constexpr int VE = 16 / (int)sizeof(E);
    static_assert(CH * D / VE % NT == 0, "whole vectors per thread");
#pragma unroll
    for (int i = 0; i < CH * D / VE / NT; ++i) {
      const int idx = threadIdx.x + i * NT, t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
      const float f = __expf(gs[t]);
      uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
      E* ke = reinterpret_cast<E*>(&kv);
#pragma unroll
      for (int e = 0; e < VE; ++e) ke[e] = (E)(f * (float)ke[e]);
      *reinterpret_cast<uint4*>(Ks + t * LD + j0) = kv;
    }
  }
  __syncthreads();

  // X^T and U^T tiles (columns j of row tile w): each lane writes four consecutive columns
  f32x4 xa[D / 16], ua[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    xa[nt] = mma_k<E, CH>(zero4(), colk(Ks, LD), 16 * nt, rowk(Ts, LDT), 16 * w);
    ua[nt] = mma_k<E, CH>(zero4(), colk(QV, LD), 16 * nt, rowk(Ts, LDT), 16 * w);
  }
  __syncthreads();
  GDR_POISON(Ks, (int)sizeof(Ks));  // Khat and V are no longer read
  GDR_POISON(QV, (int)sizeof(QV));
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    store4_t(Ks, LD, 16 * nt, 16 * w, xa[nt]);
    store4_t(QV, LD, 16 * nt, 16 * w, ua[nt]);
  }
  __syncthreads();
  s2g_full<E, CH, D, NT>(Xo + u * CH * D, D, Ks, LD);
  s2g_full<E, CH, D, NT>(Uo + u * CH * D, D, QV, LD);
}

// ---------------------------------------------------------------------------------------
// Scan: per (value-row tile, head, sequence), sequential over the sequence's chunks.
// The tile of W (BV value rows x D) lives in accumulators as W^T tiles: wave w owns key tiles
// jt = w + 4q and every value sub-tile.  Each step computes R = U - X W0^T for the tile's
// value columns, the output columns O = scale (e^g (Q W0^T) + M R) (the tile holds every
// key column of its value rows, so the output needs nothing from other tiles), records W0
// and R for the backward, and carries W_next = e^{g_n} W0 + R^T (e^{g_n-g} K).
// FULL = false is the segment-map pass (ScanSeg mode 1): no output and nothing recorded.
// RES (with FULL, Delta family and Kimi Delta Attention): also write the delta-rule residual
// r_t = v_t - v_bar_t of every token.  The chunk form's R_t is beta_t r_t (the memory gains
// R_t k_t^T), so r_t = R_t / beta_t, formed from the float32 R before it is rounded.
// ---------------------------------------------------------------------------------------
// Operands of one chunk of the forward scan, held in registers while they are in flight.
// Gated DeltaNet-2 also needs the erase gates (for the erase direction a = beta e*k) and the
// value tile's write gates and values (for b = beta w*v), and M_qk for the output.
// Kimi Delta Attention reads Kbar = e^{g_n-g} K and Qhat = e^g Q (prepared per chunk) in
// place of K and Q, and the per-key-channel decay e^{g_n} of the rows this lane holds.
template <typename E, int D, int BV, int VAR, bool FULL>
struct FwdScanOps {
  RegTile<E, CH, D, 256> x, k, q, e;
  RegTile<E, CH, BV, 256> u, vt, wt;
  RegTile<E, CH, CH, 256> m, m2;
  float g;
  uint32_t braw2;  // Gated DeltaNet-2: beta of this lane's token as loaded (0 if absent or past the end)
  f32x4 eg[D / 64];
  E braw;  // residual output: beta of this lane's token, as loaded (converted where it is used)
  // fused q/k normalisation: 1 / ||q|| of chunk row 16 w + lrow; 1 / ||k|| of that row (Gated
  // DeltaNet-2: of this lane's token)
  float rnq, rnk;
};

// QKN (delta family, Gated DeltaNet-2): q and k are normalised to unit length per token.  The
// raw rows are read and the preparation's factors Rng (1 / ||q||, 1 / ||k|| per unit) are
// applied where a row enters a product: to the output's row (Q W0^T) and to the rows of
// e^{g_n-g} R that meet K in the memory update.  Gated DeltaNet-2 folds 1 / ||k_t|| into the
// per-token scalars of the products its keys enter: beta_t of a = beta e*k and e^{g_n-g_t} beta_t
// of the write term.
template <typename E, int D, int BV, int VAR, bool FULL, bool RES, bool QKN>
__global__ __launch_bounds__(256) void k_fwd_scan(Geo geo, ScanSeg sg, const E* __restrict__ k, const E* __restrict__ Xg,
                                                  const E* __restrict__ Ug, const float* __restrict__ Gg,
                                                  const float* __restrict__ h0, E* __restrict__ Hs,
                                                  E* __restrict__ Rg, float* __restrict__ ht,
                                                  const E* __restrict__ vin, const E* __restrict__ beta,
                                                  const E* __restrict__ erase, const E* __restrict__ write,
                                                  const E* __restrict__ q, const E* __restrict__ Mg,
                                                  const E* __restrict__ M2g, E* __restrict__ o,
                                                  E* __restrict__ rout, const float* __restrict__ Rng) {
  GDR_POISON_ALL();
  constexpr int NT = 256, LD = D + pad16<E>(), LDV = BV + pad16<E>(), LDR = CH + pad16<E>();
  constexpr int NJ = D / 64, NI = BV / 16;
  constexpr bool G2 = VAR == VAR_GDN2 || VAR == VAR_GDN2L;
  constexpr bool G2L = VAR == VAR_GDN2L;  // its gates are logits
  constexpr bool KDA = VAR == VAR_KDA || VAR == VAR_GLA;  // decay per key channel, per-unit operands
  constexpr bool NOX = VAR == VAR_GLA;  // nothing erased: X = 0, so R = U (no product with W0)
  constexpr bool DEC = VAR == VAR_GATED || G2;  // scalar decay
  constexpr bool OUT_G2 = FULL && G2;
  __shared__ __align__(16) E Xs[VAR == VAR_GLA ? 8 : CH * LD];
  __shared__ __align__(16) E Ks[CH * LD];
  __shared__ __align__(16) E As[G2 ? CH * LD : 8];      // a = beta e*k (GDN-2)
  __shared__ __align__(16) E Bd[G2 ? BV * LDR : 8];     // e^{g_n-g} b^T (GDN-2)
  __shared__ __align__(16) E Bn[OUT_G2 ? CH * LDV : 8]; // b (GDN-2 output)
  __shared__ float bsh[CH];
  __shared__ float rks[QKN && (VAR == VAR_GDN2 || VAR == VAR_GDN2L) ? CH : 1];  // Gated DeltaNet-2: 1 / ||k_t||
  __shared__ __align__(16) E Us[CH * LDV];
  __shared__ __align__(16) E Ws[BV * LD];
  __shared__ __align__(16) E Rn[CH * LDV];
  // e^{g_n-g} R, row-major, read through transposing reads by the update; for bfloat16, rows
  // 64 bytes apart keep those reads free of bank conflicts
  constexpr int LDD = std::is_same<E, float>::value ? BV + 4 : 32;
  static_assert(LDD >= BV, "an R row fits");
  __shared__ __align__(16) E Rd[CH * LDD];
  __shared__ __align__(16) E Qs[FULL ? CH * LD : 8];
  __shared__ __align__(16) E Ms[FULL ? CH * LDR : 8];
  __shared__ __align__(16) E M2s[OUT_G2 ? CH * LDR : 8];
  __shared__ __align__(16) E Os[FULL ? CH * LDV : 8];
  static_assert(!RES || (FULL && !G2), "the residual output is formed by the full pass of the delta family");
  static_assert(!QKN || (VAR != VAR_KDA && VAR != VAR_GLA), "fused q/k normalisation: not the per-unit operands");
  __shared__ __align__(16) E Rr[RES ? CH * LDV : 8];  // r = R / beta for this tile's value columns
  __shared__ float gs[CH];

  constexpr int NVR = D / BV;
  int sq, h, vt;
  if (!scan_block(geo, FULL ? NVR : 2 * NVR, sq, h, vt)) return;
  const bool virt = !FULL && vt >= NVR;  // segment-map pass: rows of the segment's linear part
  const int i0 = (virt ? vt - NVR : vt) * BV;
  const SeqPos sp = seq_pos(geo, sq);
  const int w = wave_id();
  const long mem = (long)sq * geo.H + h;
  const long sbase = mem * D;  // row base of this memory in [N,H,D,D]
  const int seg = blockIdx.y;
  int c0 = 0, c1 = sp.nchunks, nseg = 1;
  if (sg.mode != 0) {
    nseg = seg_count(sg, sp.nchunks);
    if (seg >= nseg) return;
    if (!FULL && seg == nseg - 1) return;  // the last segment's map is never applied
    c0 = seg * sg.lseg;
    c1 = min(sp.nchunks, c0 + sg.lseg);
  }
  const float* init = nullptr;  // start memory (rows i, columns j); none: zero, or identity rows
  if (sg.mode == 2) init = sg.starts + (mem * sg.max_seg + seg) * D * D;
  else if (sg.mode == 0 && h0) init = h0 + sbase * D;

  f32x4 S[NJ][NI];
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

  // Chunk c + 2 is loaded while chunk c is computed (two register sets, loop unrolled by two).
  // Loads past the last chunk repeat it, so every step issues the same memory operations.
  // The loads of a step are issued in three parts (part < 0: all), each in the stretch of the
  // step whose matrix-core work hides its issue: X and U with R, Q and M with the output,
  // the keys and gates with the memory update.
  using Ops = FwdScanOps<E, D, BV, VAR, FULL>;
  auto load = [&](Ops& p, int c, int part) {
    const int cc = min(c, c1 - 1);
    const long u = (long)(sp.gc0 + cc) * geo.H + h;
    const int n = min(CH, sp.len - cc * CH);
    const long tk = tok_index(geo, sp.b, h, sp.bos + cc * CH);
    if (part <= 0) {
      if constexpr (QKN) {  // first, so that the step's wait for them waits for little else
        p.rnq = Rng[u * 2 * CH + 16 * w + lrow()];  // the row this lane holds in R^T and O^T
        p.rnk = Rng[u * 2 * CH + CH + (G2 ? (int)(threadIdx.x & (CH - 1)) : 16 * w + lrow())];
      }
      if constexpr (!NOX) p.x.load(Xg + u * CH * D, D, CH);
      p.u.load(Ug + u * CH * D + i0, D, CH);
      if constexpr (KDA) {
#pragma unroll
        for (int qq = 0; qq < NJ; ++qq) p.eg[qq] = *reinterpret_cast<const f32x4*>(Gg + u * D + acc_row(16 * (w + 4 * qq), 0));
      }
    }
    if (part < 0 || part == 1) {
      if constexpr (FULL) {
        p.q.load(q + (KDA ? u * CH : tk) * D, D, KDA ? CH : n);
        p.m.load(Mg + u * CH * CH, CH, CH);
        if constexpr (G2) p.m2.load(M2g + u * CH * CH, CH, CH);
      }
    }
    if (part < 0 || part == 2) {
      if constexpr (KDA) {
        p.k.load(k + u * CH * D, D, CH);
      } else {
        p.k.load(k + tk * D, D, n);
        p.g = Gg[u * CH + (threadIdx.x & (CH - 1))];
      }
      if constexpr (RES) {  // a plain load (valid row), no arithmetic on it until the step uses it
        const int t = min((int)(threadIdx.x & (CH - 1)), n - 1);
        p.braw = beta[tk + t];
      }
      if constexpr (G2) {
        p.e.load(erase + tk * D, D, n);
        p.vt.load(vin + tk * D + i0, D, n);
        p.wt.load(write + tk * D + i0, D, n);
        p.braw2 = load_gate_raw(beta ? beta + tk : nullptr, n, (int)(threadIdx.x & (CH - 1)));
      }
    }
  };
  auto step = [&](int c, Ops& p) {
    const long u = (long)(sp.gc0 + c) * geo.H + h;
    const int n = min(CH, sp.len - c * CH);
    const long tk = tok_index(geo, sp.b, h, sp.bos + c * CH);
    float rnq_c = 0.f, rnk_c = 0.f;  // this chunk's factors, kept before p is refilled
    if constexpr (QKN) {
      rnq_c = p.rnq;
      rnk_c = p.rnk;
    }
    if constexpr (!NOX) p.x.store(Xs, LD);
    p.k.store(Ks, LD);
    p.u.store(Us, LDV);
    if constexpr (FULL) {
      p.q.store(Qs, LD);
      p.m.store(Ms, LDR);
      if constexpr (G2) p.m2.store(M2s, LDR);
    }
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
    if constexpr (RES) {  // residual output: 1 / beta (0 past the end)
      if (threadIdx.x < CH) bsh[threadIdx.x] = ((int)threadIdx.x < n) ? 1.f / (float)p.braw : 0.f;
    }
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) store4_t(Ws, LD, 16 * (w + 4 * qq), 16 * it, S[qq][it]);
    __syncthreads();
    if constexpr (G2) {
      // a = beta e*k (row-major) and e^{g_n-g_t} b_t = e^{g_n-g_t} beta_t w_t*v_t (transposed)
      const float gn0 = gs[CH - 1];
      using RE = decltype(p.e);
      using RV = decltype(p.vt);
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
#pragma unroll
      for (int it = 0; it < RV::IT; ++it) {
        const int t = p.vt.row(it), i = p.vt.col(it);
        const float bt = virt ? 0.f : bsh[t];
        float sc = bt * __expf(gn0 - gs[t]);  // (times 1 / ||k_t||: the write term meets the raw k_t)
        if constexpr (QKN) sc *= rks[t];
        typename RV::V bnv;
        E* bn = reinterpret_cast<E*>(&bnv);
#pragma unroll
        for (int x = 0; x < RV::VE; ++x) {
          const float bv = g2_gate<G2L>((float)p.wt.elem(it, x)) * (float)p.vt.elem(it, x);
          Bd[(i + x) * LDR + t] = (E)(sc * bv);
          bn[x] = (E)(bt * bv);
        }
        if constexpr (FULL) *reinterpret_cast<typename RV::V*>(Bn + t * LDV + i) = bnv;
      }
    }
    load(p, c + 2, 0);
    const float gn = gs[CH - 1];
    // R^T = U^T - W X^T: the lane holds chunk row tl and four consecutive value columns
    const int tl = 16 * w + lrow();
    float dec = 1.f;  // e^{g_n - g_t} (times 1 / ||k_t||: the row of R that meets the raw k_t)
    if constexpr (DEC) dec = __expf(gn - gs[tl]);
    if constexpr (QKN && !G2) dec *= rnk_c;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      f32x4 acc = zero4();
      if constexpr (!NOX) acc = mma_k<E, D>(zero4(), rowk(Ws, LD), 16 * it, rowk(Xs, LD), 16 * w);
      const int c4 = 16 * it + 4 * lgrp();
      const f32x4 rv = (virt ? zero4() : get4(Us + tl * LDV + c4)) - acc;
      put4(Rn + tl * LDV + c4, rv);
      put4(Rd + tl * LDD + c4, dec * rv);
      if constexpr (RES) put4(Rr + tl * LDV + c4, bsh[tl] * rv);
    }
    if constexpr (FULL) s2g_full<E, BV, D, NT>(Hs + u * D * D + (long)i0 * D, D, Ws, LD);
    __syncthreads();
    if constexpr (FULL) {
      load(p, c + 2, 1);
      s2g_full<E, CH, BV, NT>(Rg + u * CH * D + i0, D, Rn, LDV);
      if (o) {
        // O = scale (e^g (Q W0^T) + M R [+ M_qk b]) for this tile's value columns
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          // O^T = W (e^g Q)^T + R^T M^T (+ b^T M_qk^T), four consecutive columns per lane
          const f32x4 a1 = mma_k<E, D>(zero4(), rowk(Ws, LD), 16 * it, rowk(Qs, LD), 16 * w);
          f32x4 a2 = mma_k<E, CH>(zero4(), colk(Rn, LDV), 16 * it, rowk(Ms, LDR), 16 * w);
          if constexpr (G2) a2 = mma_k<E, CH>(a2, colk(Bn, LDV), 16 * it, rowk(M2s, LDR), 16 * w);
          float e = 1.f;  // e^{g_t} (times 1 / ||q_t||: the product used the raw q_t)
          if constexpr (DEC) e = __expf(gs[tl]);
          if constexpr (QKN) e *= rnq_c;
          put4(Os + tl * LDV + 16 * it + 4 * lgrp(), geo.scale * (e * a1 + a2));
        }
      }
    }
    load(p, c + 2, 2);
    float eg = 1.f;
    if constexpr (DEC) eg = __expf(gn);
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        if constexpr (KDA) S[qq][it] *= egk[qq];
        else S[qq][it] *= eg;
        if constexpr (G2) {
          // W_next = e^{g_n} W0 + R'^T (e^{g_n-g} a) + b^T (e^{g_n-g} k)
          S[qq][it] = mma_k<E, CH>(S[qq][it], colk(As, LD), 16 * (w + 4 * qq), colk(Rd, LDD), 16 * it);
          S[qq][it] = mma_k<E, CH>(S[qq][it], colk(Ks, LD), 16 * (w + 4 * qq), rowk(Bd, LDR), 16 * it);
        } else {
          S[qq][it] = mma_k<E, CH>(S[qq][it], colk(Ks, LD), 16 * (w + 4 * qq), colk(Rd, LDD), 16 * it);
        }
      }
    __syncthreads();
    if constexpr (FULL) {
      if (o) s2g_rows<E, CH, BV, NT>(o + tk * D + i0, D, Os, LDV, n);
    }
    if constexpr (RES) s2g_rows<E, CH, BV, NT>(rout + tk * D + i0, D, Rr, LDV, n);
    GDR_POISON_ALL();  // debug builds: nothing in LDS is carried to the next step
  };
  if (c1 > c0) {
    Ops pa, pb;
    load(pa, c0, -1);
    load(pb, c0 + 1, -1);
    // Every trip of the loop runs both steps (an odd last chunk runs after it), so the
    // memory operations in flight at the top of the loop are the same on every path.
    int c = c0;
    for (; c + 1 < c1; c += 2) {
      step(c, pa);
      step(c + 1, pb);
    }
    if (c < c1) step(c, pa);
  }
  float* out = nullptr;  // final memory: ht, or this segment's map
  if (!FULL) out = sg.maps + ((mem * sg.max_seg + seg) * 2 + (virt ? 1 : 0)) * D * D;
  else if (ht && seg == nseg - 1) out = ht + sbase * D;
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
// Host launchers
// ---------------------------------------------------------------------------------------
template <typename E, int D, int VAR>
static hipError_t fwd_impl(const Plan& p, const gdr_inputs& in, void* o, void* r, float* ht, bool want_out,
                           hipStream_t st) {
  const Geo& g = p.geo;
  const dim3 cgrid(g.total_chunks, g.H);
  if (g.total_chunks > 0) {
    if constexpr (VAR == VAR_GDN2 || VAR == VAR_GDN2L) {
      const hipError_t e = launch_fwd_prep_gdn2<E, D>(p, in, st);
      if (e != hipSuccess) return e;
    } else if constexpr (VAR == VAR_KDA || VAR == VAR_GLA) {
      const hipError_t e = launch_fwd_prep_kda<E, D>(p, in, st);
      if (e != hipSuccess) return e;
    } else {
      TraceScope ts_("fwd_prep", st);
      auto prep = [&](auto kern) {
        hipLaunchKernelGGL(kern, cgrid, dim3(256), 0, st, g, (const E*)in.q, (const E*)in.k, (const E*)in.v,
                           (const E*)in.beta, (const E*)in.alpha, (E*)p.X, (E*)p.Ub, (E*)p.M, p.G, p.Li, p.Rn);
      };
      if (p.qkn) {
        if (p.gates) prep(k_fwd_prep<E, D, VAR, true, true>);
        else prep(k_fwd_prep<E, D, VAR, false, true>);
      } else {
        if (p.gates) prep(k_fwd_prep<E, D, VAR, true, false>);
        else prep(k_fwd_prep<E, D, VAR, false, false>);
      }
    }
  }
  constexpr bool KDA = VAR == VAR_KDA || VAR == VAR_GLA;
  const E* kin = KDA ? (const E*)p.Kb : (const E*)in.k;
  const E* qin = KDA ? (const E*)p.Qh : (const E*)in.q;
  const float* gin = KDA ? p.Gn : p.G;
  E* out = want_out ? (E*)o : nullptr;
  E* rout = (want_out && r) ? (E*)r : nullptr;
  auto launch = [&](auto kern, int bv, int nvm, const ScanSeg& sg, const float* h0, float* htp, E* rr) {
    hipLaunchKernelGGL(kern, dim3(scan_grid(g, nvm * D / bv), sg.mode ? sg.max_seg : 1), dim3(256), 0, st, g, sg, kin,
                       (const E*)p.X, (const E*)p.Ub, gin, h0, (E*)p.Hs, (E*)p.R, htp, (const E*)in.v,
                       (const E*)in.beta, (const E*)in.erase, (const E*)in.write, qin, (const E*)p.M, (const E*)p.M2,
                       out, rr, (const float*)p.Rn);
  };
  auto scan_q = [&](auto full, auto qkn, const ScanSeg& sg, const float* h0, float* htp) {
    constexpr bool F = decltype(full)::value;
    constexpr bool Q = decltype(qkn)::value;
    constexpr bool RES_OK = F && (VAR == VAR_DELTANET || VAR == VAR_GATED || VAR == VAR_KDA);  // residual output
    const int nvm = F ? 1 : 2;
    if (std::is_same<E, float>::value || p.bv == 16) {
      if constexpr (RES_OK) {
        if (rout) return launch(k_fwd_scan<E, D, 16, VAR, F, true, Q>, 16, nvm, sg, h0, htp, rout);
      }
      launch(k_fwd_scan<E, D, 16, VAR, F, false, Q>, 16, nvm, sg, h0, htp, nullptr);
    } else if constexpr (!std::is_same<E, float>::value) {
      if constexpr (RES_OK) {
        if (rout) return launch(k_fwd_scan<E, D, 32, VAR, F, true, Q>, 32, nvm, sg, h0, htp, rout);
      }
      launch(k_fwd_scan<E, D, 32, VAR, F, false, Q>, 32, nvm, sg, h0, htp, nullptr);
    }
  };
  auto scan = [&](auto full, const ScanSeg& sg, const float* h0, float* htp) {
    if constexpr (!KDA) {
      if (p.qkn) return scan_q(full, std::true_type{}, sg, h0, htp);
    }
    scan_q(full, std::false_type{}, sg, h0, htp);
  };
  if (p.lseg == 0) {
    TraceScope ts_("fwd_scan", st);
    scan(std::true_type{}, ScanSeg{0, 0, 1, nullptr, nullptr, 0}, in.h0, ht);
  } else {
    {
      TraceScope ts_("fwd_scan_maps", st);
      scan(std::false_type{}, ScanSeg{1, p.lseg, p.max_seg, p.seg_maps, nullptr, 0}, nullptr, nullptr);
    }
    const hipError_t e = launch_seg_combine(p, ScanSeg{0, p.lseg, p.max_seg, p.seg_maps, nullptr, 0}, in.h0, false, st);
    if (e != hipSuccess) return e;
    TraceScope ts_("fwd_scan", st);
    scan(std::true_type{}, ScanSeg{2, p.lseg, p.max_seg, nullptr, p.seg_starts, 0}, nullptr, ht);
  }
  return hipGetLastError();
}

hipError_t run_forward(const Plan& p, const gdr_inputs& in, void* o, void* r, float* ht, bool want_out,
                       hipStream_t st) {
  const bool bf = p.dtype == GDR_BF16;
#define GDR_FWD_CASE(V)                                                                  \
  if (bf && p.D == 128) return fwd_impl<bf16, 128, V>(p, in, o, r, ht, want_out, st);    \
  if (bf && p.D == 64) return fwd_impl<bf16, 64, V>(p, in, o, r, ht, want_out, st);      \
  if (!bf && p.D == 64) return fwd_impl<float, 64, V>(p, in, o, r, ht, want_out, st);    \
  break;
  switch (p.variant) {
    case GDR_DELTANET: GDR_FWD_CASE(VAR_DELTANET)
    case GDR_GATED: GDR_FWD_CASE(VAR_GATED)
    case GDR_KDA: GDR_FWD_CASE(VAR_KDA)
    case GDR_GLA: GDR_FWD_CASE(VAR_GLA)
    case GDR_GDN2:
      if (p.gates) { GDR_FWD_CASE(VAR_GDN2L) }
      GDR_FWD_CASE(VAR_GDN2)
    default: break;
  }
#undef GDR_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdr
