// Gated DeltaNet-2 chunk kernels: separate per-key-channel erase gates e and per-value-channel
// write gates w on top of a scalar decay alpha.  Token update (erase along a = beta e*k, write
// b = beta w*v at address k):  W_t = alpha_t W_{t-1} (I - k_t a_t^T) + b_t k_t^T.
//
// Chunk form (n <= 64 tokens from W0; g = in-chunk cumsum of log alpha, E_ts = e^{g_t - g_s}):
//   A_kk = tril_strict((K K^T) * E),  A_ak = tril_strict((K A^T) * E)
//   M_qk = tril((Q K^T) * E),          M_qa = tril((Q A^T) * E)
//   L = I + A_ak,  X' = L^{-1} (e^g * K),  U'' = -L^{-1} A_kk B
//   R' = U'' - X' W0^T                  (R' = -Y: minus the memory's predictions W'_t k_t)
//   O  = scale ((e^g * Q) W0^T + M_qa R' + M_qk B)
//   W_next = e^{g_n} W0 + R'^T (e^{g_n-g} * A) + B^T (e^{g_n-g} * K)
// The scans (which also write the output) are shared with the delta family (fwd.hip, bwd.hip);
// this file holds the prep kernel and the three backward stages.
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

// Rno (q/k normalisation; NULL without): q and k are scaled to unit length per token as they are
// loaded (normalize_rows) and 1/||q||, 1/||k|| are kept per unit in Rno (zero past the end); the
// scans and the backward stages scale the raw rows they load with them.
template <typename E, int D, bool LOG>
__global__ __launch_bounds__(512) void k_fwd_prep_gdn2(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                       const E* __restrict__ v, const E* __restrict__ beta,
                                                       const E* __restrict__ alpha, const E* __restrict__ erase,
                                                       const E* __restrict__ write, E* __restrict__ Xo,
                                                       E* __restrict__ Uo, E* __restrict__ U2o, E* __restrict__ Mqa,
                                                       E* __restrict__ Mqk, float* __restrict__ Go,
                                                       float* __restrict__ Lio, float* __restrict__ Akko,
                                                       float* __restrict__ Aako, float* __restrict__ Rno) {
  GDR_POISON_ALL();
  constexpr int NT = 512, NW = NT / 64, LD = D + pad16<E>(), LDT = CH + pad16<E>(), LF = CH + 4;
  constexpr int NQ = D / 32;  // column tiles per wave in the 64 x D products
  __shared__ __align__(16) E Ks[CH * LD];   // K, then e^g K, then X'
  __shared__ __align__(16) E Qs[CH * LD];   // Q, then A_kk B, then U''
  __shared__ __align__(16) E As[CH * LD];   // a = beta e*k
  __shared__ __align__(16) E Bs[CH * LD];   // b = beta w*v
  __shared__ __align__(16) E Akk[CH * LDT];
  __shared__ __align__(16) E Ti[CH * LDT];  // solve scratch, then L^{-1}
  __shared__ __align__(16) float Ls[CH * LF];
  __shared__ __align__(16) float Li[CH * LF];
  __shared__ float gs[CH], bs[CH];

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wr = w & 3, wc = w >> 2;  // 64 x D products: row tile wr, column half wc
  const int n = cp.n;

  // The gates are loaded first, as raw values (lanes past the end read 0), and staged after the
  // first tile store: waiting for them then waits for nothing the store did not already need.
  uint32_t braw = 0, araw = 0;
  if (threadIdx.x < CH) {
    braw = load_gate_raw(beta ? beta + tk : nullptr, n, threadIdx.x);
    araw = load_gate_raw(alpha + tk, n, threadIdx.x);
  }
  {
    RegTile<E, CH, D, NT> rk, re, rv, rw, rq;
    rk.load(k + tk * D, D, n);
    re.load(erase + tk * D, D, n);
    rv.load(v + tk * D, D, n);
    rw.load(write + tk * D, D, n);
    rq.load(q + tk * D, D, n);
    if (Rno) {
      normalize_rows(rk, Rno + u * 2 * CH + CH);
      normalize_rows(rq, Rno + u * 2 * CH);
    }
    rq.store(Qs, LD);
    rk.store(Ks, LD);
    if (threadIdx.x < CH) {
      const int t = threadIdx.x;
      const bool ok = t < n;
      bs[t] = ok ? (beta ? g2_gate<LOG>(gate_from_raw<E>(braw)) : 1.f) : 0.f;
      const float xa = gate_from_raw<E>(araw);
      const float la = ok ? (LOG ? gate_neg_softplus(xa) : logf(xa)) : 0.f;
      const float g = wave_incl_scan(la);
      gs[t] = g;
      Go[u * CH + t] = g;
    }
    __syncthreads();
    using RT = decltype(rk);
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
      const int t = rk.row(it), j = rk.col(it);
      typename RT::V av, bv;
      E* ae = reinterpret_cast<E*>(&av);
      E* be = reinterpret_cast<E*>(&bv);
      const float bt = bs[t];
#pragma unroll
      for (int x = 0; x < RT::VE; ++x) {
        ae[x] = (E)(bt * g2_gate<LOG>((float)re.elem(it, x)) * (float)rk.elem(it, x));
        be[x] = (E)(bt * g2_gate<LOG>((float)rw.elem(it, x)) * (float)rv.elem(it, x));
      }
      *reinterpret_cast<typename RT::V*>(As + t * LD + j) = av;
      *reinterpret_cast<typename RT::V*>(Bs + t * LD + j) = bv;
    }
  }
  __syncthreads();

  // 40 Gram tile jobs: A_kk, A_ak (strict lower), M_qk, M_qa (lower, to global).  Formed
  // transposed, so each lane holds four consecutive columns s of one row t (one vector store).
  auto put4 = [](E* dst, const float* v) {
    if constexpr (sizeof(E) == 2) *reinterpret_cast<bf16x4*>(dst) = bf16x4{(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
    else *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  };
#pragma unroll
  for (int job_r = 0; job_r < (40 + NW - 1) / NW; ++job_r) {
    const int job = w + job_r * NW;
    if (job >= 40) break;
    const int which = job / 10;
    int mt, nt;
    tri_tile(job % 10, mt, nt);
    const E* lhs = (which < 2) ? Ks : Qs;
    const E* rhs = (which == 0 || which == 2) ? Ks : As;
    const f32x4 acc = mma_k<E, D>(zero4(), rowk(rhs, LD), 16 * nt, rowk(lhs, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    float val[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + r;
      const bool keep = (which < 2) ? (s < t) : (s <= t);
      val[r] = keep ? acc[r] * __expf(gs[t] - gs[s]) : 0.f;
    }
    const float4 v4 = make_float4(val[0], val[1], val[2], val[3]);
    if (which == 0) {
      put4(Akk + t * LDT + s0, val);
      *reinterpret_cast<float4*>(Akko + (u * CH + t) * CH + s0) = v4;
    } else if (which == 1) {
      *reinterpret_cast<float4*>(Ls + t * LF + s0) = v4;
      *reinterpret_cast<float4*>(Aako + (u * CH + t) * CH + s0) = v4;
    } else {
      put4((which == 2 ? Mqk : Mqa) + (u * CH + t) * CH + s0, val);
    }
  }
#pragma unroll
  for (int idx_r = 0; idx_r < ((CH * CH / 4) + NT - 1) / NT; ++idx_r) {  // tiles above the diagonal
    const int idx = (int)threadIdx.x + idx_r * NT;
    if (idx >= CH * CH / 4) break;
    const int t = idx >> 4, s0 = (idx & 15) * 4;
    if ((s0 >> 4) > (t >> 4)) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      put4(Mqk + (u * CH + t) * CH + s0, z);
      put4(Mqa + (u * CH + t) * CH + s0, z);
      put4(Akk + t * LDT + s0, z);
      *reinterpret_cast<float4*>(Akko + (u * CH + t) * CH + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(Aako + (u * CH + t) * CH + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();
  solve_unit_lower64<NT>(Ls, LF, Li, LF, reinterpret_cast<float*>(Ti));
  s2g_full<float, CH, CH, NT>(Lio + u * CH * CH, CH, Li, LF);  // L^{-1} for the backward
#pragma unroll
  for (int idx_r = 0; idx_r < ((CH * CH / 4) + NT - 1) / NT; ++idx_r) {  // L^{-1} as an operand, four columns at a time
    const int idx = (int)threadIdx.x + idx_r * NT;
    if (idx >= CH * CH / 4) break;
    const int t = idx >> 4, s0 = (idx & 15) * 4;
    const float4 l = *reinterpret_cast<const float4*>(Li + t * LF + s0);
    const float v[4] = {s0 <= t ? l.x : 0.f, s0 + 1 <= t ? l.y : 0.f, s0 + 2 <= t ? l.z : 0.f, s0 + 3 <= t ? l.w : 0.f};
    put4(Ti + t * LDT + s0, v);
  }
  // (A_kk B)^T into registers (the Q buffer receives it below)
  f32x4 cu[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) cu[q] = mma_k<E, CH>(zero4(), colk(Bs, LD), 16 * (wc * NQ + q), rowk(Akk, LDT), 16 * wr);
  {  // Khat = e^g K in place, 16 bytes at a time
    constexpr int VE = 16 / (int)sizeof(E);
#pragma unroll
    for (int idx_r = 0; idx_r < ((CH * D / VE) + NT - 1) / NT; ++idx_r) {
      const int idx = (int)threadIdx.x + idx_r * NT;
      if (idx >= CH * D / VE) break;
      const int t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
      const float f = __expf(gs[t]);
      uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
      E* ke = reinterpret_cast<E*>(&kv);
#pragma unroll
      for (int e = 0; e < VE; ++e) ke[e] = (E)(f * (float)ke[e]);
      *reinterpret_cast<uint4*>(Ks + t * LD + j0) = kv;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) store4_t(Qs, LD, 16 * (wc * NQ + q), 16 * wr, cu[q]);
  __syncthreads();
  // X'^T and U''^T tiles: each lane writes four consecutive columns
  f32x4 xa[NQ], ua[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    xa[q] = mma_k<E, CH>(zero4(), colk(Ks, LD), 16 * nt, rowk(Ti, LDT), 16 * wr);
    ua[q] = -mma_k<E, CH>(zero4(), colk(Qs, LD), 16 * nt, rowk(Ti, LDT), 16 * wr);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    store4_t(Ks, LD, 16 * nt, 16 * wr, xa[q]);
    store4_t(Qs, LD, 16 * nt, 16 * wr, ua[q]);
  }
  __syncthreads();
  s2g_full<E, CH, D, NT>(Xo + u * CH * D, D, Ks, LD);
  s2g_full<E, CH, D, NT>(Uo + u * CH * D, D, Qs, LD);
  s2g_full<E, CH, D, NT>(U2o + u * CH * D, D, Qs, LD);
}

// ---------------------------------------------------------------------------------------
// Backward, stage 1: products with the chunk-start memory W0 and the end-of-chunk gradient dW.
//   dQhat = dO W0, dX' = -dR' W0, dAbar = R' dW, dKbar = B dW, dM_qa = dO R'^T, dM_qk = dO B^T,
//   dB_state = (e^{g_n-g} K) dW^T, and e^{g_n} <W0, dW>.   (dR' comes from the reverse scan.)
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct G2StateLds {
  static constexpr int LD = D + pad16<E>(), LDR = CH + pad16<E>();
  static constexpr int TK = CH * LD * (int)sizeof(E), TH = D * LDR * (int)sizeof(E);
  static constexpr int BYTES = 6 * TK + 2 * TH;
};

template <typename E, int D, bool LOG>
__global__ __launch_bounds__(512) void k_bwd_gdn2_state(Geo geo, const E* __restrict__ k, const E* __restrict__ v,
                                                        const E* __restrict__ beta, const E* __restrict__ erase,
                                                        const E* __restrict__ write, const E* __restrict__ dO,
                                                        const float* __restrict__ Gg, const E* __restrict__ Hs,
                                                        const E* __restrict__ Rg, const E* __restrict__ dHs,
                                                        const E* __restrict__ dRg, Plan p) {
  GDR_POISON_ALL();
  using Ly = G2StateLds<E, D>;
  constexpr int NT = 512, LD = Ly::LD, LDR = Ly::LDR, KH = 64, NH = D / KH, NQ = D / 32;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float gs[CH], bs[CH], red[NT / 64];
  __shared__ float rkb[8][CH], rab[8][CH];
  E* Ks = reinterpret_cast<E*>(smem);
  E* As = Ks + CH * LD;
  E* Bs = As + CH * LD;
  E* dOs = Bs + CH * LD;
  E* dRs = dOs + CH * LD;
  E* Rs = dRs + CH * LD;
  E* Wh = Rs + CH * LD;   // one 64-row block of W0, row-major (rows i, columns j)
  E* dWh = Wh + D * LDR;  // the same block of dW
  static_assert(KH * LD <= D * LDR, "a row-major block fits the region");

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wm = w & 3, wn = w >> 2, n = cp.n;
  // Products are formed transposed: a lane holds row t = 16 (row tile) + lrow and four
  // consecutive columns 4 lgrp .. +3 of each 16-column tile, so results go out as vectors.
  const int tr = 16 * wm + lrow();

  float graw = 0.f;  // the gates first, raw; staged after the first tile stores
  uint32_t braw = 0;
  if (threadIdx.x < CH) {
    graw = Gg[u * CH + threadIdx.x];
    braw = load_gate_raw(beta ? beta + tk : nullptr, n, threadIdx.x);
  }
  {
    RegTile<E, CH, D, NT> rk, re, rv, rw;
    float rnk[decltype(rk)::IT];  // q/k normalisation: 1 / ||k|| of the rows of rk this thread holds
    if (p.qkn) load_row_factors(rk, p.Rn + u * 2 * CH + CH, rnk);
    rk.load(k + tk * D, D, n);
    re.load(erase + tk * D, D, n);
    rv.load(v + tk * D, D, n);
    rw.load(write + tk * D, D, n);
    g2s_rows<E, CH, D, NT>(dOs, LD, dO + tk * D, D, n);
    g2s_rows<E, CH, D, NT>(Rs, LD, Rg + u * CH * D, D, CH);
    g2s_rows<E, CH, D, NT>(dRs, LD, dRg + u * CH * D, D, CH);
    if (p.qkn) scale_rows(rk, rnk);  // the keys as the preparation normalised them
    rk.store(Ks, LD);
    if (threadIdx.x < CH) {
      const int t = threadIdx.x;
      gs[t] = graw;
      bs[t] = t < n ? (beta ? g2_gate<LOG>(gate_from_raw<E>(braw)) : 1.f) : 0.f;
    }
    __syncthreads();
    using RT = decltype(rk);
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
      const int t = rk.row(it), j = rk.col(it);
      typename RT::V av, bv;
      E* ae = reinterpret_cast<E*>(&av);
      E* be = reinterpret_cast<E*>(&bv);
      const float bt = bs[t];
#pragma unroll
      for (int x = 0; x < RT::VE; ++x) {
        ae[x] = (E)(bt * g2_gate<LOG>((float)re.elem(it, x)) * (float)rk.elem(it, x));
        be[x] = (E)(bt * g2_gate<LOG>((float)rw.elem(it, x)) * (float)rv.elem(it, x));
      }
      *reinterpret_cast<typename RT::V*>(As + t * LD + j) = av;
      *reinterpret_cast<typename RT::V*>(Bs + t * LD + j) = bv;
    }
  }
  const float gn = gs[CH - 1];
  f32x4 acc1[D / 16], dab[NQ], dkb[NQ], mqa[2], mqk[2];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc1[i] = zero4();
#pragma unroll
  for (int i = 0; i < NQ; ++i) dab[i] = dkb[i] = zero4();
  mqa[0] = mqa[1] = mqk[0] = mqk[1] = zero4();
  float gam = 0.f;
  float* db1 = p.g2_db + u * CH * D;
  for (int ih = 0; ih < NH; ++ih) {
    __syncthreads();
    g2s_rows<E, KH, D, NT>(Wh, LD, Hs + u * D * D + (long)ih * KH * D, D, KH);
    g2s_rows<E, KH, D, NT>(dWh, LD, dHs + u * D * D + (long)ih * KH * D, D, KH);
    __syncthreads();
    const E* Aop = (w < 4 ? dOs : dRs) + ih * KH;
    // (dO W0)^T or (dR W0)^T: columns j, rows t
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = mma_k<E, KH>(acc1[nt], colk(Wh, LD), 16 * nt, rowk(Aop, LD), 16 * wm);
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      dab[qq] = mma_k<E, KH>(dab[qq], colk(dWh, LD), 16 * (wn * NQ + qq), rowk(Rs + ih * KH, LD), 16 * wm);
      dkb[qq] = mma_k<E, KH>(dkb[qq], colk(dWh, LD), 16 * (wn * NQ + qq), rowk(Bs + ih * KH, LD), 16 * wm);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
      mqa[e] = mma_k<E, KH>(mqa[e], rowk(Rs + ih * KH, LD), 16 * nt, rowk(dOs + ih * KH, LD), 16 * mt);
      mqk[e] = mma_k<E, KH>(mqk[e], rowk(Bs + ih * KH, LD), 16 * nt, rowk(dOs + ih * KH, LD), 16 * mt);
      // dB_state for the value columns of this block: (e^{g_n-g} K) dW^T, held transposed
      const f32x4 acc = mma_k<E, D>(zero4(), rowk(dWh, LD), 16 * nt, rowk(Ks, LD), 16 * mt);
      const int t = 16 * mt + lrow();
      put4(db1 + t * D + ih * KH + 16 * nt + 4 * lgrp(), __expf(gn - gs[t]) * acc);
    }
    {  // <W0, dW> over this block, 16 bytes at a time
      constexpr int VE = 16 / (int)sizeof(E);
#pragma unroll
      for (int idx_r = 0; idx_r < ((KH * D / VE) + NT - 1) / NT; ++idx_r) {
        const int idx = (int)threadIdx.x + idx_r * NT;
        if (idx >= KH * D / VE) break;
        const int i = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
        const uint4 a = *reinterpret_cast<const uint4*>(Wh + i * LD + j0);
        const uint4 c = *reinterpret_cast<const uint4*>(dWh + i * LD + j0);
        const E* ae = reinterpret_cast<const E*>(&a);
        const E* ce = reinterpret_cast<const E*>(&c);
#pragma unroll
        for (int e = 0; e < VE; ++e) gam += (float)ae[e] * (float)ce[e];
      }
    }
  }
  float* dq1 = p.g2_dq + u * CH * D;
  float* dx = p.g2_dx + u * CH * D;
  {
    const float f = (w < 4) ? geo.scale * __expf(gs[tr]) : -1.f;
    float* dst = (w < 4 ? dq1 : dx) + tr * D + 4 * lgrp();
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) put4(dst + 16 * nt, f * acc1[nt]);
  }
  {
    float* dk1 = p.g2_dk + u * CH * D;
    float* da1 = p.g2_da + u * CH * D;
    const float dec = __expf(gn - gs[tr]);
    float pk = 0.f, pa = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int j0 = 16 * (wn * NQ + qq) + 4 * lgrp();
      const f32x4 xk = dec * dkb[qq], xa = dec * dab[qq];
      put4(dk1 + tr * D + j0, xk);
      put4(da1 + tr * D + j0, xa);
      const f32x4 kk = get4(Ks + tr * LD + j0), aa = get4(As + tr * LD + j0);
      pk += kk[0] * xk[0] + kk[1] * xk[1] + kk[2] * xk[2] + kk[3] * xk[3];
      pa += aa[0] * xa[0] + aa[1] * xa[1] + aa[2] * xa[2] + aa[3] * xa[3];
    }
    pk = sum_rows4(pk);
    pa = sum_rows4(pa);
    if (lgrp() == 0) {
      rkb[w][tr] = pk;
      rab[w][tr] = pa;
    }
  }
  float* dmqa = p.g2_dmqa + u * CH * CH;
  float* dmqk = p.g2_dmqk + u * CH * CH;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    f32x4 xa, xk;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = s0 + r <= t;
      xa[r] = keep ? geo.scale * mqa[e][r] : 0.f;
      xk[r] = keep ? geo.scale * mqk[e][r] : 0.f;
    }
    put4(dmqa + t * CH + s0, xa);
    put4(dmqk + t * CH + s0, xk);
  }
  gam = wave_sum(gam);
  if (lane_id() == 0) red[w] = gam;
  __syncthreads();
  if (threadIdx.x < CH) {
    const int t = threadIdx.x, b0 = t >> 4;
    float* rows = p.g2_rows + u * 4 * CH;
    rows[t] = rkb[b0][t] + rkb[b0 + 4][t] + rab[b0][t] + rab[b0 + 4][t];
    if (t == 0) {
      float g4 = 0.f;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) g4 += red[i];
      rows[3 * CH] = __expf(gn) * g4;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Backward, stage 2: the solve side.  With A_kk and L^{-1} as the forward computed them,
//   dKhat = L^-T dX',  dC = -L^-T dR',  dA_ak = tril_strict(-dKhat X'^T + dC U''^T),
//   dA_kk = tril_strict(dC B^T),  dB = dB_state + A_kk^T dC + M_qk^T dO,
//   dv = beta w*dB, dw = beta v*dB;  dk += e^g dKhat.
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct G2WyLds {
  static constexpr int LD = D + pad16<E>(), LDT = CH + pad16<E>();
  static constexpr int TK = CH * LD * (int)sizeof(E), SQ = CH * LDT * (int)sizeof(E);
  static constexpr int BYTES = TK + 3 * SQ + 4 * TK;
};

template <typename E, int D, bool LOG>
__global__ __launch_bounds__(512) void k_bwd_gdn2_wy(Geo geo, const E* __restrict__ k, const E* __restrict__ v,
                                                     const E* __restrict__ beta, const E* __restrict__ erase,
                                                     const E* __restrict__ write, const E* __restrict__ dO,
                                                     const float* __restrict__ Gg, const E* __restrict__ Xg,
                                                     const E* __restrict__ U2g, const E* __restrict__ M2g,
                                                     const E* __restrict__ dRg, E* __restrict__ dv,
                                                     E* __restrict__ dw, Plan p) {
  GDR_POISON_ALL();
  using Ly = G2WyLds<E, D>;
  constexpr int NT = 512, NW = NT / 64, LD = Ly::LD, LDT = Ly::LDT, NQ = D / 32;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float gs[CH], bs[CH], rk[NW][CH], rb[NW][CH];  // row sums, one part per wave
  E* Ks = reinterpret_cast<E*>(smem);
  E* LiN = Ks + CH * LD;  // L^{-1}, row-major (read k-major where its transpose is needed)
  E* AkkE = LiN + CH * LDT;
  E* Mqk = AkkE + CH * LDT;
  char* un = reinterpret_cast<char*>(Mqk + CH * LDT);
  E* P1 = reinterpret_cast<E*>(un);
  E* P2 = P1 + CH * LD;
  E* P3 = P2 + CH * LD;
  E* P4 = P3 + CH * LD;

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wr = w & 3, wc = w >> 2, n = cp.n;
  // Products below are formed transposed: lane (lrow, lgrp) of wave w holds row t = 16 (w & 3)
  // + lrow and four consecutive columns 4 lgrp .. +3 of each of its 16-column tiles (half of
  // them: tiles NQ (w >> 2) ..), so every global or LDS access of a result is one vector access.
  const int tr = 16 * wr + lrow();

  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    gs[t] = Gg[u * CH + t];
    bs[t] = t < n ? (beta ? g2_gate<LOG>((float)beta[tk + t]) : 1.f) : 0.f;
  }
  g2s_rows_scaled<E, CH, D, NT>(Ks, LD, k + tk * D, D, n, p.qkn ? p.Rn + u * 2 * CH + CH : nullptr);
  g2s_rows<E, CH, CH, NT>(Mqk, LDT, M2g + u * CH * CH, CH, CH);
  {  // L^{-1} and A_kk as the forward computed them
    RegTile<float, CH, CH, NT> rli, rakk;
    rli.load(p.Li + u * CH * CH, CH, CH);
    rakk.load(p.A1 + u * CH * CH, CH, CH);
    static_assert(decltype(rli)::VE == 4, "four floats per vector");
#pragma unroll
    for (int it = 0; it < decltype(rli)::IT; ++it) {
      const int t = rli.row(it), s0 = rli.col(it);
      put4(LiN + t * LDT + s0, f32x4{rli.elem(it, 0), rli.elem(it, 1), rli.elem(it, 2), rli.elem(it, 3)});
      put4(AkkE + t * LDT + s0, f32x4{rakk.elem(it, 0), rakk.elem(it, 1), rakk.elem(it, 2), rakk.elem(it, 3)});
    }
  }
  {  // dX' (float32 workspace) and dR' into the union region
    const float* dx = p.g2_dx + u * CH * D;
#pragma unroll
    for (int idx_r = 0; idx_r < ((CH * D / 4) + NT - 1) / NT; ++idx_r) {
      const int idx = (int)threadIdx.x + idx_r * NT;
      if (idx >= CH * D / 4) break;
      const int t = idx / (D / 4), j0 = (idx % (D / 4)) * 4;
      const float4 x = *reinterpret_cast<const float4*>(dx + t * D + j0);
      put4(P1 + t * LD + j0, f32x4{x.x, x.y, x.z, x.w});
    }
    g2s_rows<E, CH, D, NT>(P2, LD, dRg + u * CH * D, D, CH);
  }
  __syncthreads();
  // dKhat^T = dX'^T L^{-1} and dC^T = -dR'^T L^{-1} (columns j, rows t)
  f32x4 dkh[NQ], dc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    dkh[q] = mma_k<E, CH>(zero4(), colk(P1, LD), 16 * nt, colk(LiN, LDT), 16 * wr);
    dc[q] = -mma_k<E, CH>(zero4(), colk(P2, LD), 16 * nt, colk(LiN, LDT), 16 * wr);
  }
  __syncthreads();
  {
    float* dk1 = p.g2_dk + u * CH * D;
    const float et = __expf(gs[tr]);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int nt = wc * NQ + q;
      store4_t(P1, LD, 16 * nt, 16 * wr, dkh[q]);
      store4_t(P2, LD, 16 * nt, 16 * wr, dc[q]);
      const int j0 = 16 * nt + 4 * lgrp();
      const f32x4 x = et * dkh[q];
      float4 d = *reinterpret_cast<const float4*>(dk1 + tr * D + j0);
      d.x += x[0]; d.y += x[1]; d.z += x[2]; d.w += x[3];
      *reinterpret_cast<float4*>(dk1 + tr * D + j0) = d;
      const f32x4 kv = get4(Ks + tr * LD + j0);
      part += kv[0] * x[0] + kv[1] * x[1] + kv[2] * x[2] + kv[3] * x[3];
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rk[w][tr] = part;
  }
  g2s_rows<E, CH, D, NT>(P3, LD, Xg + u * CH * D, D, CH);
  g2s_rows<E, CH, D, NT>(P4, LD, U2g + u * CH * D, D, CH);
  __syncthreads();
  float* daak = p.g2_daak + u * CH * CH;
#pragma unroll
  for (int id_r = 0; id_r < (16 + NW - 1) / NW; ++id_r) {
    const int id = w + id_r * NW;
    if (id >= 16) break;
    const int mt = id >> 2, nt = id & 3;
    f32x4 acc = mma_k<E, D>(zero4(), rowk(P4, LD), 16 * nt, rowk(P2, LD), 16 * mt);
    acc = acc - mma_k<E, D>(zero4(), rowk(P3, LD), 16 * nt, rowk(P1, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (s0 + r < t) ? acc[r] : 0.f;
    put4(daak + t * CH + s0, acc);
  }
  __syncthreads();
  {  // b = beta w*v into P3, dO into P4
    RegTile<E, CH, D, NT> rv, rw;
    rv.load(v + tk * D, D, n);
    rw.load(write + tk * D, D, n);
    using RT = decltype(rv);
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
      const int t = rv.row(it), i = rv.col(it);
      typename RT::V bv;
      E* be = reinterpret_cast<E*>(&bv);
      const float bt = bs[t];
#pragma unroll
      for (int x = 0; x < RT::VE; ++x) be[x] = (E)(bt * g2_gate<LOG>((float)rw.elem(it, x)) * (float)rv.elem(it, x));
      *reinterpret_cast<typename RT::V*>(P3 + t * LD + i) = bv;
    }
    g2s_rows<E, CH, D, NT>(P4, LD, dO + tk * D, D, n);
  }
  __syncthreads();
  float* dakk = p.g2_dakk + u * CH * CH;
#pragma unroll
  for (int id_r = 0; id_r < (16 + NW - 1) / NW; ++id_r) {
    const int id = w + id_r * NW;
    if (id >= 16) break;
    const int mt = id >> 2, nt = id & 3;
    f32x4 acc = mma_k<E, D>(zero4(), rowk(P3, LD), 16 * nt, rowk(P2, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (s0 + r < t) ? acc[r] : 0.f;
    put4(dakk + t * CH + s0, acc);
  }
  // dB^T = dB_state^T + dC^T A_kk + (scale dO)^T M_qk
  f32x4 dbt[NQ];
  const float* db1 = p.g2_db + u * CH * D;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    f32x4 a = mma_k<E, CH>(zero4(), colk(P2, LD), 16 * nt, colk(AkkE, LDT), 16 * wr);
    const f32x4 bq = mma_k<E, CH>(zero4(), colk(P4, LD), 16 * nt, colk(Mqk, LDT), 16 * wr);
    const float4 d = *reinterpret_cast<const float4*>(db1 + tr * D + 16 * nt + 4 * lgrp());
    a[0] += geo.scale * bq[0] + d.x;
    a[1] += geo.scale * bq[1] + d.y;
    a[2] += geo.scale * bq[2] + d.z;
    a[3] += geo.scale * bq[3] + d.w;
    dbt[q] = a;
  }
  __syncthreads();
  {  // v and w into P1 / P3 for the gate products; outputs staged through P2 / P4
    g2s_rows<E, CH, D, NT>(P1, LD, v + tk * D, D, n);
    g2s_rows<E, CH, D, NT>(P3, LD, write + tk * D, D, n);
  }
  __syncthreads();
  {
    const float bt = bs[tr];
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int nt = wc * NQ + q;
      const int i0 = 16 * nt + 4 * lgrp();
      const f32x4 vv = get4(P1 + tr * LD + i0);
      f32x4 ww = get4(P3 + tr * LD + i0);
      if constexpr (LOG) {
#pragma unroll
        for (int x = 0; x < 4; ++x) ww[x] = gate_sigmoid(ww[x]);
      }
      const f32x4 ov = bt * ww * dbt[q];
      f32x4 ow = bt * vv * dbt[q];
      if constexpr (LOG) ow *= ww * (1.f - ww);  // gradient w.r.t. the write-gate logit
      part += ww[0] * vv[0] * dbt[q][0] + ww[1] * vv[1] * dbt[q][1] + ww[2] * vv[2] * dbt[q][2] + ww[3] * vv[3] * dbt[q][3];
      store4_t(P2, LD, 16 * nt, 16 * wr, ov);
      store4_t(P4, LD, 16 * nt, 16 * wr, ow);
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rb[w][tr] = part;
  }
  __syncthreads();
  s2g_rows<E, CH, D, NT>(dv + tk * D, D, P2, LD, n);
  s2g_rows<E, CH, D, NT>(dw + tk * D, D, P4, LD, n);
  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    float* rows = p.g2_rows + u * 4 * CH;
    rows[CH + t] = rk[t >> 4][t] + rk[(t >> 4) + 4][t];
    rows[2 * CH + t] = rb[t >> 4][t] + rb[(t >> 4) + 4][t];
  }
}

// ---------------------------------------------------------------------------------------
// Backward, stage 3: Gram slots, gates and the decay gradient.
//   dk += At_kk K + At_kk^T K + At_ak A + Mt_qk^T Q,  dq += Mt_qk K + Mt_qa A,
//   da += At_ak^T K + Mt_qa^T Q   (At = dA * E, Mt = dM * E),
//   de = beta da*k, dk += beta da*e, dbeta += sum(da*e*k) + sum(dB*w*v),
//   d log alpha_t = rectangle + suffix + prefix sums + e^{g_n} <W0, dW>;  dalpha = that / alpha.
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct G2GramLds {
  static constexpr int LD = D + pad16<E>(), LDT = CH + pad16<E>(), LF = CH + 4;
  static constexpr int TK = CH * LD * (int)sizeof(E), SQ = CH * LDT * (int)sizeof(E), F = CH * LF * 4;
  static constexpr int BYTES = 4 * TK + 4 * SQ + F;
};

template <typename E, int D, bool LOG>
__global__ __launch_bounds__(512) void k_bwd_gdn2_gram(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                       const E* __restrict__ beta, const E* __restrict__ alpha,
                                                       const E* __restrict__ erase, const float* __restrict__ Gg,
                                                       const E* __restrict__ Mqag, const E* __restrict__ Mqkg,
                                                       E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dbeta,
                                                       E* __restrict__ dalpha, E* __restrict__ derase, Plan p) {
  GDR_POISON_ALL();
  using Ly = G2GramLds<E, D>;
  constexpr int NT = 512, NW = NT / 64, LD = Ly::LD, LDT = Ly::LDT, LF = Ly::LF, NQ = D / 32;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float gs[CH], bs[CH], rq[NW][CH], re_[NW][CH];  // row sums, one part per wave
  __shared__ float rkn[2][CH], rqn[2][CH];  // q/k normalisation: k~ . dk~, q~ . dq~, one part per column half
  E* Ks = reinterpret_cast<E*>(smem);
  E* As = Ks + CH * LD;
  E* Qs = As + CH * LD;
  E* Es = Qs + CH * LD;
  E* Tkk = Es + CH * LD;
  E* Tak = Tkk + CH * LDT;
  E* Tqk = Tak + CH * LDT;
  E* Tqa = Tqk + CH * LDT;
  float* Pair = reinterpret_cast<float*>(Tqa + CH * LDT);

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wr = w & 3, wc = w >> 2, n = cp.n;

  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    gs[t] = Gg[u * CH + t];
    bs[t] = t < n ? (beta ? g2_gate<LOG>((float)beta[tk + t]) : 1.f) : 0.f;
  }
  g2s_rows_scaled<E, CH, D, NT>(Ks, LD, k + tk * D, D, n, p.qkn ? p.Rn + u * 2 * CH + CH : nullptr);
  g2s_rows_scaled<E, CH, D, NT>(Qs, LD, q + tk * D, D, n, p.qkn ? p.Rn + u * 2 * CH : nullptr);
  g2s_rows<E, CH, D, NT>(Es, LD, erase + tk * D, D, n);
  // Products are formed transposed: lane (lrow, lgrp) of wave w holds row t = 16 (w & 3) + lrow
  // and four consecutive columns 4 lgrp .. +3 of each of its 16-column tiles (half of them:
  // tiles NQ (w >> 2) ..), so every access of a result is one vector access.
  const int tr = 16 * wr + lrow();
  f32x4 aq[NQ], ak[NQ], aa[NQ];
  float rnq = 0.f, rnk = 0.f;  // q/k normalisation: 1 / ||q||, 1 / ||k|| of row tr
  if (p.qkn) {
    rnq = p.Rn[u * 2 * CH + tr];
    rnk = p.Rn[u * 2 * CH + CH + tr];
  }
  {  // the partial gradients from the earlier stages, issued early
    const float* dq1 = p.g2_dq + u * CH * D + tr * D + 4 * lgrp();
    const float* dk1 = p.g2_dk + u * CH * D + tr * D + 4 * lgrp();
    const float* da1 = p.g2_da + u * CH * D + tr * D + 4 * lgrp();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int nt = wc * NQ + q;
      const float4 x = *reinterpret_cast<const float4*>(dq1 + 16 * nt);
      const float4 y = *reinterpret_cast<const float4*>(dk1 + 16 * nt);
      const float4 z = *reinterpret_cast<const float4*>(da1 + 16 * nt);
      aq[q] = f32x4{x.x, x.y, x.z, x.w};
      ak[q] = f32x4{y.x, y.y, y.z, y.w};
      aa[q] = f32x4{z.x, z.y, z.z, z.w};
    }
  }
  __syncthreads();
  {  // a = beta e*k, 16 bytes at a time
    constexpr int VE = 16 / (int)sizeof(E);
#pragma unroll
    for (int idx_r = 0; idx_r < ((CH * D / VE) + NT - 1) / NT; ++idx_r) {
      const int idx = (int)threadIdx.x + idx_r * NT;
      if (idx >= CH * D / VE) break;
      const int t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
      const uint4 ev = *reinterpret_cast<const uint4*>(Es + t * LD + j0);
      const uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
      const E* ee = reinterpret_cast<const E*>(&ev);
      const E* ke = reinterpret_cast<const E*>(&kv);
      uint4 av;
      E* ae = reinterpret_cast<E*>(&av);
      const float bt = bs[t];
      uint4 gv;  // the erase gates themselves (sigmoid of the logits when logits are given)
      E* ge = reinterpret_cast<E*>(&gv);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float ev_ = g2_gate<LOG>((float)ee[e]);
        ge[e] = (E)ev_;
        ae[e] = (E)(bt * ev_ * (float)ke[e]);
      }
      *reinterpret_cast<uint4*>(As + t * LD + j0) = av;
      if constexpr (LOG) *reinterpret_cast<uint4*>(Es + t * LD + j0) = gv;
    }
  }
  {  // decayed gradients of the chunk matrices and the pair terms, four columns at a time
    const long o0 = u * CH * CH;
#pragma unroll
    for (int idx_r = 0; idx_r < ((CH * CH / 4) + NT - 1) / NT; ++idx_r) {
      const int idx = (int)threadIdx.x + idx_r * NT;
      if (idx >= CH * CH / 4) break;
      const int t = idx >> 4, s0 = (idx & 15) * 4;
      const long o = o0 + t * CH + s0;
      const float4 d1 = *reinterpret_cast<const float4*>(p.g2_dakk + o);
      const float4 d2 = *reinterpret_cast<const float4*>(p.g2_daak + o);
      const float4 d3 = *reinterpret_cast<const float4*>(p.g2_dmqk + o);
      const float4 d4 = *reinterpret_cast<const float4*>(p.g2_dmqa + o);
      const float4 a1 = *reinterpret_cast<const float4*>(p.A1 + o);
      const float4 a2 = *reinterpret_cast<const float4*>(p.A2 + o);
      const f32x4 m1 = get4(Mqkg + o), m2 = get4(Mqag + o);
      const float e1[4] = {d1.x, d1.y, d1.z, d1.w}, e2[4] = {d2.x, d2.y, d2.z, d2.w};
      const float e3[4] = {d3.x, d3.y, d3.z, d3.w}, e4[4] = {d4.x, d4.y, d4.z, d4.w};
      const float f1[4] = {a1.x, a1.y, a1.z, a1.w}, f2[4] = {a2.x, a2.y, a2.z, a2.w};
      f32x4 tkk, tak, tqk, tqa, pr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s2 = s0 + r;
        const float dec = (s2 <= t) ? __expf(gs[t] - gs[s2]) : 0.f;
        tkk[r] = e1[r] * dec;
        tak[r] = e2[r] * dec;
        tqk[r] = e3[r] * dec;
        tqa[r] = e4[r] * dec;
        pr[r] = (s2 < t) ? e1[r] * f1[r] + e2[r] * f2[r] + e3[r] * m1[r] + e4[r] * m2[r] : 0.f;
      }
      put4(Tkk + t * LDT + s0, tkk);
      put4(Tak + t * LDT + s0, tak);
      put4(Tqk + t * LDT + s0, tqk);
      put4(Tqa + t * LDT + s0, tqa);
      put4(Pair + t * LF + s0, pr);
    }
  }
  __syncthreads();
  {
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const f32x4 qv = get4(Qs + tr * LD + 16 * (wc * NQ + q) + 4 * lgrp());
      part += qv[0] * aq[q][0] + qv[1] * aq[q][1] + qv[2] * aq[q][2] + qv[3] * aq[q][3];
    }
    part = sum_rows4(part);
    if (lgrp() == 0) rq[w][tr] = part;
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    ak[q] = mma_k<E, CH>(ak[q], colk(Ks, LD), 16 * nt, rowk(Tkk, LDT), 16 * wr);
    ak[q] = mma_k<E, CH>(ak[q], colk(Ks, LD), 16 * nt, colk(Tkk, LDT), 16 * wr);
    ak[q] = mma_k<E, CH>(ak[q], colk(As, LD), 16 * nt, rowk(Tak, LDT), 16 * wr);
    ak[q] = mma_k<E, CH>(ak[q], colk(Qs, LD), 16 * nt, colk(Tqk, LDT), 16 * wr);
    aq[q] = mma_k<E, CH>(aq[q], colk(Ks, LD), 16 * nt, rowk(Tqk, LDT), 16 * wr);
    aq[q] = mma_k<E, CH>(aq[q], colk(As, LD), 16 * nt, rowk(Tqa, LDT), 16 * wr);
    aa[q] = mma_k<E, CH>(aa[q], colk(Ks, LD), 16 * nt, colk(Tak, LDT), 16 * wr);
    aa[q] = mma_k<E, CH>(aa[q], colk(Qs, LD), 16 * nt, colk(Tqa, LDT), 16 * wr);
  }
  // gates: de = beta da*k, dk += beta da*e, dbeta_a = sum_j da*e*k
  {
    const float bt = bs[tr];
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j0 = 16 * (wc * NQ + q) + 4 * lgrp();
      const f32x4 kk = get4(Ks + tr * LD + j0), ee = get4(Es + tr * LD + j0), da = aa[q];
      ak[q] += bt * da * ee;
      part += da[0] * ee[0] * kk[0] + da[1] * ee[1] * kk[1] + da[2] * ee[2] * kk[2] + da[3] * ee[3] * kk[3];
      aa[q] = bt * da * kk;  // now de
      if constexpr (LOG) aa[q] *= ee * (1.f - ee);  // w.r.t. the erase-gate logit
    }
    part = sum_rows4(part);
    if (lgrp() == 0) re_[w][tr] = part;
  }
  if (p.qkn) {  // dq~, dk~ are complete: x~ . dx~ over this wave's columns of row tr (a row's
    // columns are split over waves w and w ^ 4), summed after the next barrier
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j0 = 16 * (wc * NQ + q) + 4 * lgrp();
      const f32x4 kv = get4(Ks + tr * LD + j0), qv = get4(Qs + tr * LD + j0);
      pk += kv[0] * ak[q][0] + kv[1] * ak[q][1] + kv[2] * ak[q][2] + kv[3] * ak[q][3];
      pq += qv[0] * aq[q][0] + qv[1] * aq[q][1] + qv[2] * aq[q][2] + qv[3] * aq[q][3];
    }
    pk = sum_rows4(pk);
    pq = sum_rows4(pq);
    if (lgrp() == 0) {
      rkn[wc][tr] = pk;
      rqn[wc][tr] = pq;
    }
  }
  // prefix sums along each row of the pair terms: lanes over columns, rows over the waves
#pragma unroll
  for (int uu_r = 0; uu_r < ((CH) + (NT / 64) - 1) / (NT / 64); ++uu_r) {
    const int uu = w + uu_r * (NT / 64);
    if (uu >= CH) break;
    float* row = Pair + uu * LF;
    row[lane_id()] = wave_incl_scan(row[lane_id()]);
  }
  __syncthreads();
  if (p.qkn) {  // w.r.t. the raw rows: dx = (dx~ - x~ (x~ . dx~)) / ||x||, in float32; each lane
    // reads only the elements of K and Q it overwrites below
    const float dk_ = rkn[0][tr] + rkn[1][tr], dq_ = rqn[0][tr] + rqn[1][tr];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j0 = 16 * (wc * NQ + q) + 4 * lgrp();
      ak[q] = (ak[q] - dk_ * get4(Ks + tr * LD + j0)) * rnk;
      aq[q] = (aq[q] - dq_ * get4(Qs + tr * LD + j0)) * rnq;
    }
  }
  // outputs through LDS (K, A, Q regions are free now)
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    store4_t(Ks, LD, 16 * nt, 16 * wr, ak[q]);
    store4_t(Qs, LD, 16 * nt, 16 * wr, aq[q]);
    store4_t(As, LD, 16 * nt, 16 * wr, aa[q]);
  }
  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    const float* rows = p.g2_rows + u * 4 * CH;
    float rect = 0.f;
    if (t > 0) {
#pragma unroll 16
      for (int uu = 0; uu < CH; ++uu) rect += (uu >= t) ? Pair[uu * LF + t - 1] : 0.f;
    }
    const int tq = CH - 1 - t;
    const float suf_r = wave_incl_scan(rq[tq >> 4][tq] + rq[(tq >> 4) + 4][tq] + rows[CH + tq]);
    const float suf = __shfl(suf_r, CH - 1 - t, 64);
    const float inc = wave_incl_scan(rows[t]);
    float pre = __shfl_up(inc, 1, 64);
    if (t == 0) pre = 0.f;
    const float dla = rect + suf + pre + rows[3 * CH];
    if (t < n) {
      if constexpr (LOG) {  // w.r.t. the logits: d log alpha (-sigmoid(x_alpha)), dbeta beta (1 - beta)
        dalpha[tk + t] = (E)(-dla * gate_sigmoid((float)alpha[tk + t]));
        if (dbeta) dbeta[tk + t] = (E)((rows[2 * CH + t] + re_[t >> 4][t] + re_[(t >> 4) + 4][t]) * bs[t] * (1.f - bs[t]));
      } else {
        dalpha[tk + t] = (E)(dla / (float)alpha[tk + t]);
        if (dbeta) dbeta[tk + t] = (E)(rows[2 * CH + t] + re_[t >> 4][t] + re_[(t >> 4) + 4][t]);
      }
    }
  }
  __syncthreads();
  s2g_rows<E, CH, D, NT>(dk + tk * D, D, Ks, LD, n);
  s2g_rows<E, CH, D, NT>(dq + tk * D, D, Qs, LD, n);
  s2g_rows<E, CH, D, NT>(derase + tk * D, D, As, LD, n);
}

template <typename E, int D, bool LOG>
static hipError_t bwd_gdn2_impl(const Plan& p, const gdr_inputs& in, const void* dO, const gdr_grads& gr,
                                hipStream_t st) {
  const dim3 grid(p.geo.total_chunks, p.geo.H);
  {
    TraceScope ts_("bwd_gdn2_state", st);
    hipLaunchKernelGGL((k_bwd_gdn2_state<E, D, LOG>), grid, dim3(512), 0, st, p.geo, (const E*)in.k, (const E*)in.v,
                       (const E*)in.beta, (const E*)in.erase, (const E*)in.write, (const E*)dO, (const float*)p.G,
                       (const E*)p.Hs, (const E*)p.R, (const E*)p.dHs, (const E*)p.dR, p);
  }
  {
    TraceScope ts_("bwd_gdn2_wy", st);
    hipLaunchKernelGGL((k_bwd_gdn2_wy<E, D, LOG>), grid, dim3(512), 0, st, p.geo, (const E*)in.k, (const E*)in.v,
                       (const E*)in.beta, (const E*)in.erase, (const E*)in.write, (const E*)dO, (const float*)p.G,
                       (const E*)p.X, (const E*)p.U2, (const E*)p.M2, (const E*)p.dR, (E*)gr.dv, (E*)gr.dwrite, p);
  }
  {
    TraceScope ts_("bwd_gdn2_gram", st);
    hipLaunchKernelGGL((k_bwd_gdn2_gram<E, D, LOG>), grid, dim3(512), 0, st, p.geo, (const E*)in.q, (const E*)in.k,
                       (const E*)in.beta, (const E*)in.alpha, (const E*)in.erase, (const float*)p.G, (const E*)p.M,
                       (const E*)p.M2, (E*)gr.dq, (E*)gr.dk, (E*)gr.dbeta, (E*)gr.dalpha, (E*)gr.derase, p);
  }
  return hipGetLastError();
}
template <typename E, int D>
hipError_t launch_bwd_gdn2(const Plan& p, const gdr_inputs& in, const void* dO, const gdr_grads& gr, hipStream_t st) {
  return p.gates ? bwd_gdn2_impl<E, D, true>(p, in, dO, gr, st) : bwd_gdn2_impl<E, D, false>(p, in, dO, gr, st);
}
template hipError_t launch_bwd_gdn2<bf16, 128>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);
template hipError_t launch_bwd_gdn2<bf16, 64>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);
template hipError_t launch_bwd_gdn2<float, 64>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);

template <typename E, int D>
hipError_t launch_fwd_prep_gdn2(const Plan& p, const gdr_inputs& in, hipStream_t st) {
  TraceScope ts_("fwd_prep_gdn2", st);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(p.geo.total_chunks, p.geo.H), dim3(512), 0, st, p.geo, (const E*)in.q,
                       (const E*)in.k, (const E*)in.v, (const E*)in.beta, (const E*)in.alpha, (const E*)in.erase,
                       (const E*)in.write, (E*)p.X, (E*)p.Ub, (E*)p.U2, (E*)p.M, (E*)p.M2, p.G, p.Li, p.A1, p.A2,
                       p.qkn ? p.Rn : nullptr);
  };
  if (p.gates) go(k_fwd_prep_gdn2<E, D, true>);
  else go(k_fwd_prep_gdn2<E, D, false>);
  return hipGetLastError();
}
template hipError_t launch_fwd_prep_gdn2<bf16, 128>(const Plan&, const gdr_inputs&, hipStream_t);
template hipError_t launch_fwd_prep_gdn2<bf16, 64>(const Plan&, const gdr_inputs&, hipStream_t);
template hipError_t launch_fwd_prep_gdn2<float, 64>(const Plan&, const gdr_inputs&, hipStream_t);

}  // namespace gdr
