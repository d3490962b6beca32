// Kimi Delta Attention chunk kernels: the decay alpha_t is a vector over the key channels,
// W_t = W_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
//
// Chunk form (n <= 64 tokens from W0; g_t = in-chunk cumsum of log alpha, one value per
// key channel j; all products below are per channel):
//   A_ts = sum_j k_tj k_sj e^{g_tj - g_sj} (s < t),  M_ts = sum_j q_tj k_sj e^{g_tj - g_sj} (s <= t)
//   L = I + diag(beta) A,  T = L^{-1} diag(beta),  X = T (e^g * K),  U = T V
//   R = U - X W0^T,  O = scale ((e^g * Q) W0^T + M R),  W_next = W0 diag(e^{g_n}) + R^T (e^{g_n - g} * K)
// The per-channel factor e^{g_t - g_s} cannot be pulled out of the sum over j, and e^{-g}
// overflows over a chunk, so the Grams are taken in 16-token blocks with a reference token
// between the two indices: e^{g_t - g_s} = e^{g_t - g_r} e^{g_r - g_s}.  For blocks below
// the diagonal both factors are <= 1; a diagonal block uses its first token as reference,
// which keeps the factors in range unless the block's decay is stronger than e^{-60} in some
// channel -- those (rare) diagonal blocks are summed exactly, one exponential per term.
//
// The erase-free memory with the same per-channel decay (GLA form, W <- W diag(alpha) + beta v k^T)
// is this chunk form with nothing erased: A = 0, L = I, X = 0 and R = U = diag(beta) V.  Its
// kernels are these with EF = true: the preparation forms only M (no key Gram, no solve), the
// scans skip X, the state stage skips dX, a short stage replaces the solve side (dV = beta dR,
// dbeta = sum v dR) and the Gram stage has no dA slot.
// The forward scan (which also writes the output) is the delta family's (fwd.hip) fed with
// Kbar = e^{g_n - g} * K and Qhat = e^g * Q from the prep kernel and a per-row decay of the
// carried memory.  The backward is the reverse scan (bwd.hip) and three chunk stages here.
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

namespace {
// Largest in-block decay (natural log) for which the block-start reference is used.
constexpr float KDA_REF_LIMIT = -60.f;
constexpr int cmax(int a, int b) { return a > b ? a : b; }
}  // namespace

// The float32 64 x D partial gradients handed between the backward stages (dQhat, dX, dKbar,
// dKhat) are stored tile by tile in the matrix-core accumulator layout: 16 x 16 tile (rt, ct) of
// a unit at floats ((rt * D/16 + ct) * 64 + lane) * 4, the lane's four values being rows
// 16 rt + 4 lgrp .. +3 of column 16 ct + lrow.  A tile is then one 16-byte store or load per
// lane, where row-major storage took four scattered 4-byte accesses per lane.
template <int D>
__device__ __forceinline__ int frag_off(int rt, int ct) { return ((rt * (D / 16) + ct) * 64 + lane_id()) * 4; }

// g for JW channels from a tile of alpha already loaded (rows >= n taken as log 1 = 0):
// Gs[t*ldg + j] = sum_{u<=t} log alpha_{u,j}.  Each column is one wave's inclusive scan over its
// 64 lanes (lane = token), the same arithmetic in every kernel, so all of them see the same
// values of g.  Ends with a block barrier.
// LOG: the tile holds logits x, log alpha = -softplus(x).
template <typename E, int JW, int NT, bool LOG>
__device__ void kda_cumlog(const RegTile<E, CH, JW, NT>& ra, int n, float* Gs, int ldg) {
#pragma unroll
  for (int it = 0; it < RegTile<E, CH, JW, NT>::IT; ++it) {
    if (RegTile<E, CH, JW, NT>::TOTAL % NT == 0 || threadIdx.x + it * NT < RegTile<E, CH, JW, NT>::TOTAL) {
      const int t = ra.row(it), j = ra.col(it);
#pragma unroll
      for (int x = 0; x < RegTile<E, CH, JW, NT>::VE; ++x) {
        const float a = (float)ra.elem(it, x);
        Gs[t * ldg + j + x] = (t < n) ? (LOG ? gate_neg_softplus(a) : logf(a)) : 0.f;
      }
    }
  }
  __syncthreads();
  constexpr int NW = NT / 64;
  static_assert(JW % NW == 0, "whole columns per wave");
  const int w = wave_id(), l = lane_id();
#pragma unroll
  for (int i = 0; i < JW / NW; ++i) {
    const int j = w + i * NW;
    Gs[l * ldg + j] = wave_incl_scan(Gs[l * ldg + j]);
  }
  __syncthreads();
}

// unsafe[b] = 1 when some channel decays by more than e^{KDA_REF_LIMIT} inside block b.
template <int D, int NT>
__device__ void kda_flags(const float* Gs, int ldg, int* unsafe) {
  for (int idx = threadIdx.x; idx < 4 * D; idx += NT) {
    const int b = idx / D, j = idx % D;
    if (Gs[(16 * b + 15) * ldg + j] - Gs[16 * b * ldg + j] < KDA_REF_LIMIT) unsafe[b] = 1;
  }
  __syncthreads();
}

// The chunk's Grams.  Inputs in LDS: Ks (K), Kr = K e^{g - g_ref} and, WITH_M, Qr = Q e^{g - g_ref}
// (ref = the first token of the row's 16-token block), Gs, unsafe flags; Cl is scratch.
// Outputs: Ls[t][s] = lsc_t A_ts below the diagonal, optionally (Af != NULL) Af[t*ldaf + s] = A_ts
// (zero on and above the diagonal), Mo[t][s] = M_ts (global, zero above the diagonal).
// qg: Q in global memory (token rows, used only for exact diagonal blocks); qinv, if not NULL,
// 1 / ||q|| per row, with which those rows are scaled as normalize_rows scaled the tile's.
// Ends with a barrier.  WITH_A = false (nothing erased): M only; Ls and Af are not touched.
template <typename E, int D, int NT, bool WITH_M, bool WITH_A = true>
__device__ void kda_grams(const E* Ks, const E* Qr, const E* Kr, E* Cl, const float* Gs, const int* unsafe,
                          float* Ls, const float* lsc, float* Af, int ldaf, E* Mo, const E* qg, int n,
                          const float* qinv) {
  static_assert(WITH_A || WITH_M, "at least one Gram");
  constexpr int LD = D + pad16<E>(), LDG = D + 4, LF = CH + 4;
  const int w = wave_id();
  for (int I = 0; I < 4; ++I) {
    const int ref = 16 * I;
    const bool uns = unsafe[I] != 0;
    // column operand of row block I: K_s e^{g_ref - g_s} for s < ref + 16, 16 bytes at a time
    constexpr int VE = 16 / (int)sizeof(E);
    for (int idx = threadIdx.x; idx < (ref + 16) * (D / VE); idx += NT) {
      const int s = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
      const uint4 kv = *reinterpret_cast<const uint4*>(Ks + s * LD + j0);
      const E* ke = reinterpret_cast<const E*>(&kv);
      uint4 cv;
      E* ce = reinterpret_cast<E*>(&cv);
      const bool zero = uns && s >= ref;
#pragma unroll
      for (int e = 0; e < VE; ++e)
        ce[e] = (E)(zero ? 0.f : (float)ke[e] * __expf(Gs[ref * LDG + j0 + e] - Gs[s * LDG + j0 + e]));
      *reinterpret_cast<uint4*>(Cl + s * LD + j0) = cv;
    }
    __syncthreads();
    // Tiles (row block I, column block J <= I), formed transposed so each lane holds four
    // consecutive columns s of one row t and writes them with one vector store.
    const int njobs = (WITH_A && WITH_M ? 2 : 1) * (I + 1);
    for (int job = w; job < njobs; job += NT / 64) {
      const bool isM = WITH_A ? job > I : true;
      const int J = (WITH_A && isM) ? job - I - 1 : job;
      if (J == I && uns) continue;
      const f32x4 acc = mma_k<E, D>(zero4(), rowk(Cl, LD), 16 * J, rowk(isM ? Qr : Kr, LD), ref);
      const int t = ref + lrow(), s0 = 16 * J + 4 * lgrp();
      if (isM) {
        if constexpr (WITH_M) {
          E m[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) m[r] = (E)((s0 + r <= t) ? acc[r] : 0.f);
          if constexpr (sizeof(E) == 2) {
            *reinterpret_cast<bf16x4*>(Mo + t * CH + s0) = bf16x4{m[0], m[1], m[2], m[3]};
          } else {
            *reinterpret_cast<float4*>(Mo + t * CH + s0) = make_float4(m[0], m[1], m[2], m[3]);
          }
        }
      } else {
        float4 a;
        a.x = (s0 < t) ? acc[0] : 0.f;
        a.y = (s0 + 1 < t) ? acc[1] : 0.f;
        a.z = (s0 + 2 < t) ? acc[2] : 0.f;
        a.w = (s0 + 3 < t) ? acc[3] : 0.f;
        const float l = lsc[t];
        *reinterpret_cast<float4*>(Ls + t * LF + s0) = make_float4(l * a.x, l * a.y, l * a.z, l * a.w);
        if (Af) *reinterpret_cast<float4*>(Af + t * ldaf + s0) = a;
      }
    }
    __syncthreads();
  }
  // blocks above the diagonal are zero
  for (int idx = threadIdx.x; idx < CH * CH / 4; idx += NT) {
    const int t = idx >> 4, s0 = (idx & 15) * 4;
    if (s0 >= 16 * ((t >> 4) + 1)) {
      if (Af) *reinterpret_cast<float4*>(Af + t * ldaf + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (WITH_M) {
        if constexpr (sizeof(E) == 2) *reinterpret_cast<bf16x4*>(Mo + t * CH + s0) = bf16x4{(E)0.f, (E)0.f, (E)0.f, (E)0.f};
        else *reinterpret_cast<float4*>(Mo + t * CH + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  if (unsafe[0] | unsafe[1] | unsafe[2] | unsafe[3]) {
    // upper triangles of the diagonal blocks summed exactly below (the products wrote the others)
    for (int idx = threadIdx.x; idx < 4 * 256; idx += NT) {
      const int I = idx >> 8, t = 16 * I + ((idx >> 4) & 15), s = 16 * I + (idx & 15);
      if (!unsafe[I] || s <= t) continue;
      if (Af) Af[t * ldaf + s] = 0.f;
      if constexpr (WITH_M) Mo[t * CH + s] = (E)0.f;
    }
    // exact diagonal blocks: one exponential per (t, s, j)
    for (int idx = threadIdx.x; idx < 4 * 136; idx += NT) {
      const int I = idx / 136;
      if (!unsafe[I]) continue;
      int p = idx % 136, tt = 0;
      while (p > tt) {
        p -= tt + 1;
        ++tt;
      }
      const int t = 16 * I + tt, s = 16 * I + p;
      float a = 0.f, m = 0.f;
      for (int j = 0; j < D; ++j) {
        const float e = __expf(Gs[t * LDG + j] - Gs[s * LDG + j]);
        const float ks = (float)Ks[s * LD + j];
        a += (float)Ks[t * LD + j] * ks * e;
        if constexpr (WITH_M) {
          float qv = t < n ? (float)qg[(long)t * D + j] : 0.f;
          if (qinv) qv = (float)(E)(qv * qinv[t]);
          m += qv * ks * e;
        }
      }
      if constexpr (WITH_A) {
        if (s < t) {
          Ls[t * LF + s] = lsc[t] * a;
          if (Af) Af[t * ldaf + s] = a;
        } else if (Af) {
          Af[t * ldaf + s] = 0.f;
        }
      }
      if constexpr (WITH_M) Mo[t * CH + s] = (E)m;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Forward prep: per (chunk, head).  g, Kbar, Qhat, e^{g_n}, M, L^{-1}, X, U.
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct KdaPrepLds {
  static constexpr int LD = D + pad16<E>(), LDG = D + 4, LF = CH + 4, LDT = CH + pad16<E>();
  static constexpr int TK = CH * LD * (int)sizeof(E), GB = CH * LDG * 4, F = CH * LF * 4;
  // G | Kr | Cl | K (then e^g K, then X) | Q (then Qr, then V, then U) | Ls
  static constexpr int oG = 0, oKr = GB, oCl = GB + TK, oK = GB + 2 * TK, oQ = GB + 3 * TK;
  static constexpr int oL = GB + 4 * TK, BYTES = oL + F;
  // after the Grams: L^{-1} (float) and T = L^{-1} diag(beta) over the G / Kr / Cl regions
  static constexpr int oLi = 0, oT = F;
  static_assert(F + CH * LDT * (int)sizeof(E) <= GB + 2 * TK, "L^{-1} and T must fit the freed regions");
  static_assert(CH * LDT * (int)sizeof(E) >= 4 * 256 * 4, "T doubles as the solve's scratch");
};

// LOG: beta and alpha are logits (beta = sigmoid(x), log alpha = -softplus(x) per channel).
// EF: nothing erased (see the top of this file); beta may be NULL (1).
// Rno (q/k normalisation; NULL without): q and k are scaled to unit length per token as they are
// loaded (normalize_rows), so Kbar, Qhat and every product here take the normalised rows, and
// 1/||q||, 1/||k|| are kept per unit in Rno (zero past the end) for the backward stages, which
// scale the raw rows they load with them.
template <typename E, int D, bool LOG, bool EF>
__global__ __launch_bounds__(512) void k_fwd_prep_kda(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                      const E* __restrict__ v, const E* __restrict__ beta,
                                                      const E* __restrict__ alpha, E* __restrict__ Xo,
                                                      E* __restrict__ Uo, E* __restrict__ Mo, E* __restrict__ Kbo,
                                                      E* __restrict__ Qho, float* __restrict__ Gno,
                                                      float* __restrict__ Lio, float* __restrict__ Ao,
                                                      float* __restrict__ Rno) {
  GDR_POISON_ALL();
  using Ly = KdaPrepLds<E, D>;
  constexpr int NT = 512, LD = Ly::LD, LDG = Ly::LDG, LF = Ly::LF, LDT = Ly::LDT;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float bs[CH];
  __shared__ float rnq[CH];  // Rno given: 1 / ||q|| per token
  __shared__ int unsafe[4];
  float* Gs = reinterpret_cast<float*>(smem + Ly::oG);
  E* Kr = reinterpret_cast<E*>(smem + Ly::oKr);
  E* Cl = reinterpret_cast<E*>(smem + Ly::oCl);
  E* Ks = reinterpret_cast<E*>(smem + Ly::oK);
  E* Qs = reinterpret_cast<E*>(smem + Ly::oQ);
  float* Ls = reinterpret_cast<float*>(smem + Ly::oL);

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), n = cp.n;

  // beta is loaded before the tiles (raw) and staged after K and Q are: its wait then covers
  // nothing those stores did not need, where loaded after V it would also wait for V.
  const uint32_t braw = threadIdx.x < CH ? load_gate_raw(beta ? beta + tk : nullptr, n, threadIdx.x) : 0u;
  RegTile<E, CH, D, NT> rv, rk, rq, ra;
  ra.load(alpha + tk * D, D, n);
  rk.load(k + tk * D, D, n);
  rq.load(q + tk * D, D, n);
  rv.load(v + tk * D, D, n);
  if (threadIdx.x < 4) unsafe[threadIdx.x] = 0;
  if (Rno) {  // q and k scaled to unit length per token; 1 / ||k|| straight to Rno, 1 / ||q|| via LDS
    normalize_rows(rq, rnq);
    normalize_rows(rk, Rno + u * 2 * CH + CH);
  }
  rk.store(Ks, LD);
  rq.store(Qs, LD);
  if (threadIdx.x < CH) {
    float b = gate_from_raw<E>(braw);  // 0 past the end
    if (LOG && (int)threadIdx.x < n) b = gate_sigmoid(b);
    if (EF && !beta) b = (int)threadIdx.x < n ? 1.f : 0.f;
    bs[threadIdx.x] = b;
  }
  kda_cumlog<E, D, NT, LOG>(ra, n, Gs, LDG);
  if (Rno && threadIdx.x < CH) Rno[u * 2 * CH + threadIdx.x] = rnq[threadIdx.x];
  kda_flags<D, NT>(Gs, LDG, unsafe);

  // Kbar and Qhat for the scans, e^{g_n} per channel, and the row
  // operands of the Grams (Q's buffer is overwritten in place by Qr).
  E* kb = Kbo + u * CH * D;
  E* qh = Qho + u * CH * D;
  constexpr int VE = 16 / (int)sizeof(E);
  for (int idx = threadIdx.x; idx < CH * D / VE; idx += NT) {
    const int t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
    const uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
    const uint4 qv = *reinterpret_cast<const uint4*>(Qs + t * LD + j0);
    const E* ke = reinterpret_cast<const E*>(&kv);
    const E* qe = reinterpret_cast<const E*>(&qv);
    uint4 kbv, qhv, krv, qrv;
    E* kbe = reinterpret_cast<E*>(&kbv);
    E* qhe = reinterpret_cast<E*>(&qhv);
    E* kre = reinterpret_cast<E*>(&krv);
    E* qre = reinterpret_cast<E*>(&qrv);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int j = j0 + e;
      const float g = Gs[t * LDG + j], gn = Gs[(CH - 1) * LDG + j], gb = Gs[(t & ~15) * LDG + j];
      const float kk = (float)ke[e], qq = (float)qe[e];
      kbe[e] = (E)(kk * __expf(gn - g));
      qhe[e] = (E)(qq * __expf(g));
      const float f = __expf(g - gb);
      kre[e] = (E)(kk * f);
      qre[e] = (E)(qq * f);
    }
    *reinterpret_cast<uint4*>(kb + t * D + j0) = kbv;
    *reinterpret_cast<uint4*>(qh + t * D + j0) = qhv;
    *reinterpret_cast<uint4*>(Kr + t * LD + j0) = krv;
    *reinterpret_cast<uint4*>(Qs + t * LD + j0) = qrv;
  }
  if (threadIdx.x < D) Gno[u * D + threadIdx.x] = __expf(Gs[(CH - 1) * LDG + threadIdx.x]);
  __syncthreads();
  E* Mc = Mo + u * CH * CH;
  if constexpr (EF) {
    // M only; nothing erased, so L = I and U = diag(beta) V (rows past the end load as zero)
    kda_grams<E, D, NT, true, false>(Ks, Qs, Kr, Cl, Gs, unsafe, nullptr, bs, nullptr, CH, Mc, q + tk * D, n,
                                     Rno ? rnq : nullptr);
    using RV = decltype(rv);
#pragma unroll
    for (int it = 0; it < RV::IT; ++it) {
      if (RV::TOTAL % NT == 0 || threadIdx.x + it * NT < RV::TOTAL) {
        E* e = reinterpret_cast<E*>(&rv.v[it]);
        const float b = bs[rv.row(it)];
#pragma unroll
        for (int x = 0; x < RV::VE; ++x) e[x] = (E)(b * (float)e[x]);
      }
    }
    rv.store_global(Uo + u * CH * D, D);
    return;
  }
  kda_grams<E, D, NT, true>(Ks, Qs, Kr, Cl, Gs, unsafe, Ls, bs, Ao + u * CH * CH, CH, Mc, q + tk * D, n,
                            Rno ? rnq : nullptr);

  // Khat = e^g K in place; V into the Q buffer
  for (int idx = threadIdx.x; idx < CH * D / VE; idx += NT) {
    const int t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
    uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
    E* ke = reinterpret_cast<E*>(&kv);
#pragma unroll
    for (int e = 0; e < VE; ++e) ke[e] = (E)((float)ke[e] * __expf(Gs[t * LDG + j0 + e]));
    *reinterpret_cast<uint4*>(Ks + t * LD + j0) = kv;
  }
  rv.store(Qs, LD);
  __syncthreads();
  float* Li = reinterpret_cast<float*>(smem + Ly::oLi);
  E* Ts = reinterpret_cast<E*>(smem + Ly::oT);
  solve_unit_lower64<NT>(Ls, LF, Li, LF, reinterpret_cast<float*>(Ts));
  s2g_full<float, CH, CH, NT>(Lio + u * CH * CH, CH, Li, LF);  // L^{-1} for the backward
  for (int idx = threadIdx.x; idx < CH * CH; idx += NT) {
    const int t = idx >> 6, s = idx & 63;
    Ts[t * LDT + s] = (E)(s <= t ? Li[t * LF + s] * bs[s] : 0.f);
  }
  __syncthreads();
  // X = T Khat, U = T V: wave w takes row tile w & 3 and half of the column tiles
  constexpr int NQ = D / 32;
  const int wr = w & 3, wc = w >> 2;
  f32x4 xa[NQ], ua[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    xa[q] = mma_k<E, CH>(zero4(), rowk(Ts, LDT), 16 * wr, colk(Ks, LD), 16 * nt);
    ua[q] = mma_k<E, CH>(zero4(), rowk(Ts, LDT), 16 * wr, colk(Qs, LD), 16 * nt);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nt = wc * NQ + q;
    store4_n(Ks, LD, 16 * wr, 16 * nt, xa[q]);
    store4_n(Qs, LD, 16 * wr, 16 * nt, ua[q]);
  }
  __syncthreads();
  s2g_full<E, CH, D, NT>(Xo + u * CH * D, D, Ks, LD);
  s2g_full<E, CH, D, NT>(Uo + u * CH * D, D, Qs, LD);
}

// ---------------------------------------------------------------------------------------
// Backward, stage 1: products with W0 and dW (dR from the reverse scan).
//   dQhat = scale dO W0,  dX = -dR W0,  dKbar = R dW,  dM = scale tril(dO R^T),
//   gamma_j = e^{g_nj} sum_i W0_ij dW_ij   (float32 workspace)
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct KdaStateLds {
  static constexpr int LD = D + pad16<E>(), LDR = CH + pad16<E>();
  static constexpr int TK = CH * LD * (int)sizeof(E), TH = D * LDR * (int)sizeof(E);
  static constexpr int BYTES = 3 * TK + 2 * TH;
};

// EF: nothing erased, no dX (waves 4-7 form only dKbar and dM).
template <typename E, int D, bool EF>
__global__ __launch_bounds__(512) void k_bwd_kda_state(Geo geo, const E* __restrict__ dO, const float* __restrict__ Gn,
                                                       const E* __restrict__ Hs, const E* __restrict__ Rg,
                                                       const E* __restrict__ dHs, const E* __restrict__ dRg, Plan p) {
  GDR_POISON_ALL();
  using Ly = KdaStateLds<E, D>;
  constexpr int NT = 512, LD = Ly::LD, LDR = Ly::LDR, KH = 64, NH = D / KH, NQ = D / 32, NP = NT / D;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float gpart[NP][D];
  E* dOs = reinterpret_cast<E*>(smem);
  E* Rs = dOs + CH * LD;
  E* dRs = Rs + CH * LD;
  E* Wh = dRs + CH * LD;
  E* dWh = Wh + D * LDR;

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), wm = w & 3, wn = w >> 2, n = cp.n;

  g2s_rows<E, CH, D, NT>(dOs, LD, dO + tk * D, D, n);
  g2s_rows<E, CH, D, NT>(Rs, LD, Rg + u * CH * D, D, CH);
  if constexpr (!EF) g2s_rows<E, CH, D, NT>(dRs, LD, dRg + u * CH * D, D, CH);
  f32x4 acc1[D / 16], dkb[NQ], mq[2];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc1[i] = zero4();
#pragma unroll
  for (int i = 0; i < NQ; ++i) dkb[i] = zero4();
  mq[0] = mq[1] = zero4();
  const int gj = threadIdx.x % D, gp = threadIdx.x / D;
  float gam = 0.f;
  for (int ih = 0; ih < NH; ++ih) {
    __syncthreads();
    g2s_rows_t<E, KH, D, NT>(Wh, LDR, Hs + u * D * D + (long)ih * KH * D, D, KH);
    g2s_rows_t<E, KH, D, NT>(dWh, LDR, dHs + u * D * D + (long)ih * KH * D, D, KH);
    __syncthreads();
    const E* Aop = (w < 4 ? dOs : dRs) + ih * KH;
    if (!EF || w < 4) {
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) acc1[nt] = mma_k<E, KH>(acc1[nt], rowk(Aop, LD), 16 * wm, rowk(Wh, LDR), 16 * nt);
    }
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq)
      dkb[qq] = mma_k<E, KH>(dkb[qq], rowk(Rs + ih * KH, LD), 16 * wm, rowk(dWh, LDR), 16 * (wn * NQ + qq));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int id = w + 8 * e;
      mq[e] = mma_k<E, KH>(mq[e], rowk(Rs + ih * KH, LD), 16 * (id & 3), rowk(dOs + ih * KH, LD), 16 * (id >> 2));  // dM^T
    }
    for (int i = gp; i < KH; i += NP) gam += (float)Wh[gj * LDR + i] * (float)dWh[gj * LDR + i];
  }
  gpart[gp][gj] = gam;
  float* dqh = p.kd_dqh + u * CH * D;
  float* dx = p.kd_dx + u * CH * D;
  float* dk1 = p.kd_dkb + u * CH * D;
  E* dm = reinterpret_cast<E*>(p.kd_dm) + u * CH * CH;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    if (w < 4) *reinterpret_cast<f32x4*>(dqh + frag_off<D>(wm, nt)) = geo.scale * acc1[nt];
    else if (!EF) *reinterpret_cast<f32x4*>(dx + frag_off<D>(wm, nt)) = -acc1[nt];
  }
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) *reinterpret_cast<f32x4*>(dk1 + frag_off<D>(wm, wn * NQ + qq)) = dkb[qq];
#pragma unroll
  for (int e = 0; e < 2; ++e) {  // tile (rows mt, columns nt) held transposed: four consecutive columns of row t
    const int id = w + 8 * e, mt = id >> 2, nt = id & 3;
    const int t = acc_col(16 * mt), s0 = acc_row(16 * nt, 0);
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (s0 + r <= t) ? geo.scale * mq[e][r] : 0.f;
    put4(dm + t * CH + s0, x);
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) s += gpart[i][threadIdx.x];
    p.kd_gam[u * D + threadIdx.x] = Gn[u * D + threadIdx.x] * s;
  }
}

// ---------------------------------------------------------------------------------------
// Backward, stage 2: the solve side.  With A and L^{-1} as the forward computed them (and g
// recomputed for Khat = e^g K),
//   dT = dR V^T + dX Khat^T,  dV = T^T dR,  dKhat = T^T dX,  dbeta_s = sum_t dT_ts Linv_ts,
//   dL = -strictlower(L^-T (dT diag beta) L^-T),  dbeta_t += sum_s dL_ts A_ts,  dA = diag(beta) dL.
// ---------------------------------------------------------------------------------------
template <typename E, int D>
struct KdaWyLds {
  static constexpr int LD = D + pad16<E>(), LDG = D + 4, LF = CH + 4;
  static constexpr int TK = CH * LD * (int)sizeof(E), GB = CH * LDG * 4, F = CH * LF * 4;
  // region 1: G while Khat is formed, then L^{-1} | dT | V | dR
  static constexpr int R1 = cmax(GB, 2 * F + 2 * TK);
  static constexpr int oG = 0;
  static constexpr int oLi = 0, odT = F, oV = 2 * F, odR = 2 * F + TK;
  static constexpr int oK = R1, oL = R1 + TK, oA = oL + F, odX = oA + F, END = odX + TK;
  // bfloat16 copies of L^{-1} and T = L^{-1} diag(beta) as matrix-core operands (the float32
  // path reads L^{-1} directly)
  static constexpr bool BCOPY = !std::is_same<E, float>::value;
  static constexpr int LDT = CH + pad16<E>(), SQ = CH * LDT * (int)sizeof(E);
  static constexpr int oLb = END, oTb = END + SQ, BYTES = END + (BCOPY ? 2 * SQ : 0);
};

// LOG: beta and alpha are logits; dbeta is returned w.r.t. the logit (times beta (1 - beta)).
template <typename E, int D, bool LOG>
__global__ __launch_bounds__(512) void k_bwd_kda_wy(Geo geo, const E* __restrict__ k, const E* __restrict__ v,
                                                    const E* __restrict__ beta, const E* __restrict__ alpha,
                                                    const E* __restrict__ dRg, E* __restrict__ dv,
                                                    E* __restrict__ dbeta, Plan p) {
  GDR_POISON_ALL();
  using Ly = KdaWyLds<E, D>;
  constexpr int NT = 512, LD = Ly::LD, LDG = Ly::LDG, LF = Ly::LF, NW = NT / 64;
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ __align__(16) float bs[CH];
  constexpr int PS = 4;  // threads per row or column in the beta-gradient sums (the first four waves)
  __shared__ float partc[PS][CH], partr[PS][CH];
  float* Gs = reinterpret_cast<float*>(smem + Ly::oG);
  E* Ks = reinterpret_cast<E*>(smem + Ly::oK);
  float* Ls = reinterpret_cast<float*>(smem + Ly::oL);
  float* Af = reinterpret_cast<float*>(smem + Ly::oA);
  E* dXs = reinterpret_cast<E*>(smem + Ly::odX);

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), n = cp.n;

  const uint32_t braw = threadIdx.x < CH ? load_gate_raw(beta + tk, n, threadIdx.x) : 0u;  // staged after K
  RegTile<E, CH, D, NT> rv, rdr, rk, ra;
  // dX tiles of this wave (row tile w & 3, half of the column tiles), in the hand-off layout
  constexpr int NQ = D / 32;
  const int wr = w & 3, wc = w >> 2;
  f32x4 xf[NQ];
  RegTile<float, CH, CH, NT> rli, raf;
  float rnk[decltype(rk)::IT];  // q/k normalisation: 1 / ||k|| of the rows of rk this thread holds
  if (p.qkn) load_row_factors(rk, p.Rn + u * 2 * CH + CH, rnk);
  ra.load(alpha + tk * D, D, n);
  rk.load(k + tk * D, D, n);
  rv.load(v + tk * D, D, n);
  rdr.load(dRg + u * CH * D, D, CH);
#pragma unroll
  for (int q = 0; q < NQ; ++q) xf[q] = *reinterpret_cast<const f32x4*>(p.kd_dx + u * CH * D + frag_off<D>(wr, wc * NQ + q));
  rli.load(p.Li + u * CH * CH, CH, CH);
  raf.load(p.A1 + u * CH * CH, CH, CH);
  if (p.qkn) scale_rows(rk, rnk);  // the keys as the preparation normalised them
  rk.store(Ks, LD);
  if (threadIdx.x < CH) {
    const float b = gate_from_raw<E>(braw);  // 0 past the end
    bs[threadIdx.x] = (LOG && threadIdx.x < n) ? gate_sigmoid(b) : b;
  }
  kda_cumlog<E, D, NT, LOG>(ra, n, Gs, LDG);
  {  // Khat = e^g K in place, 16 bytes at a time
    constexpr int VE = 16 / (int)sizeof(E);
    for (int idx = threadIdx.x; idx < CH * D / VE; idx += NT) {
      const int t = idx / (D / VE), j0 = (idx % (D / VE)) * VE;
      uint4 kv = *reinterpret_cast<const uint4*>(Ks + t * LD + j0);
      E* ke = reinterpret_cast<E*>(&kv);
#pragma unroll
      for (int e = 0; e < VE; ++e) ke[e] = (E)((float)ke[e] * __expf(Gs[t * LDG + j0 + e]));
      *reinterpret_cast<uint4*>(Ks + t * LD + j0) = kv;
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) store4_n(dXs, LD, 16 * wr, 16 * (wc * NQ + q), xf[q]);
  raf.store(Af, LF);
  __syncthreads();  // G is free from here on
  float* Li = reinterpret_cast<float*>(smem + Ly::oLi);
  float* dTs = reinterpret_cast<float*>(smem + Ly::odT);
  E* Vs = reinterpret_cast<E*>(smem + Ly::oV);
  E* dRs = reinterpret_cast<E*>(smem + Ly::odR);
  rli.store(Li, LF);
  rv.store(Vs, LD);
  rdr.store(dRs, LD);
  constexpr int LDT = Ly::LDT;
  E* Lb = reinterpret_cast<E*>(smem + Ly::oLb);
  E* Tb = reinterpret_cast<E*>(smem + Ly::oTb);
  if constexpr (Ly::BCOPY) {  // from the registers: L^{-1} and L^{-1} diag(beta) in bfloat16
    using RL = decltype(rli);
    static_assert(RL::VE == 4, "four floats per vector");
#pragma unroll
    for (int it = 0; it < RL::IT; ++it) {
      const int t = rli.row(it), s0 = rli.col(it);
      const f32x4 l = {rli.elem(it, 0), rli.elem(it, 1), rli.elem(it, 2), rli.elem(it, 3)};
      const float4 b4 = *reinterpret_cast<const float4*>(bs + s0);
      put4(Lb + t * LDT + s0, l);
      put4(Tb + t * LDT + s0, l * f32x4{b4.x, b4.y, b4.z, b4.w});
    }
  }
  const auto LiRow = [&]() { if constexpr (Ly::BCOPY) return rowk(Lb, LDT); else return rowk(Li, LF); }();
  const auto LiCol = [&]() { if constexpr (Ly::BCOPY) return colk(Lb, LDT); else return colk(Li, LF); }();
  __syncthreads();
  // dT^T tiles (columns s, rows t), four consecutive columns per lane
#pragma unroll
  for (int e = 0; e < 16 / NW; ++e) {
    const int id = w + NW * e, mt = id >> 2, nt = id & 3;
    const f32x4 a = mma_k<E, D>(zero4(), rowk(Vs, LD), 16 * nt, rowk(dRs, LD), 16 * mt);
    const f32x4 bb = mma_k<E, D>(zero4(), rowk(Ks, LD), 16 * nt, rowk(dXs, LD), 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (s0 + r <= t) ? a[r] + bb[r] : 0.f;
    put4(dTs + t * LF + s0, x);
  }
  const auto Tt = [&]() { if constexpr (Ly::BCOPY) return colk(Tb, LDT); else return TtView{Li, LF, bs}; }();
  // dV^T (columns j, rows t) and dKhat (rows t, columns j, in the hand-off layout): wave w takes
  // row tile w & 3 and half of the column tiles
  f32x4 dva[NQ];
  {
    float* dkh = p.kd_dkh + u * CH * D;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int nt = wc * NQ + q;
      dva[q] = mma_k<E, CH>(zero4(), colk(dRs, LD), 16 * nt, Tt, 16 * wr);
      *reinterpret_cast<f32x4*>(dkh + frag_off<D>(wr, nt)) = mma_k<E, CH>(zero4(), Tt, 16 * wr, colk(dXs, LD), 16 * nt);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) store4_t(Vs, LD, 16 * (wc * NQ + q), 16 * wr, dva[q]);
  if (threadIdx.x < PS * CH) {  // dbeta from T = Linv diag(beta): column sums
    const int s = threadIdx.x & (CH - 1), pt = threadIdx.x >> 6;
    float a = 0.f;
#pragma unroll
    for (int t = pt; t < CH; t += PS) a += dTs[t * LF + s] * Li[t * LF + s];
    partc[pt][s] = a;
  }
  __syncthreads();
  s2g_rows<E, CH, D, NT>(dv + tk * D, D, Vs, LD, n);
  // the gradient w.r.t. Linv is dT diag(beta): Pt = (dT diag(beta)) Linv^T
  float* Pt = Ls;  // L is no longer needed
#pragma unroll
  for (int e = 0; e < 16 / NW; ++e) {
    const int id = w + NW * e, mt = id >> 2, nt = id & 3;
    const f32x4 acc = mma_k<E, CH>(zero4(), RowKScaled{dTs, LF, bs}, 16 * mt, LiRow, 16 * nt);
    store4_t(Pt, LF, 16 * mt, 16 * nt, acc);
  }
  __syncthreads();
  // dL (strictly lower), transposed: dT is no longer read, so dL overwrites it in place
  E* da = reinterpret_cast<E*>(p.kd_da) + u * CH * CH;
#pragma unroll
  for (int e = 0; e < 16 / NW; ++e) {
    const int id = w + NW * e, mt = id >> 2, nt = id & 3;
    const f32x4 acc = mma_k<E, CH>(zero4(), rowk(Pt, LF), 16 * nt, LiCol, 16 * mt);
    const int t = 16 * mt + lrow(), s0 = 16 * nt + 4 * lgrp();
    f32x4 dl;
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[r] = (s0 + r < t) ? -acc[r] : 0.f;
    put4(dTs + t * LF + s0, dl);
    put4(da + t * CH + s0, bs[t] * dl);
  }
  __syncthreads();
  if (threadIdx.x < PS * CH) {  // dbeta from L = I + diag(beta) A: row sums
    const int t = threadIdx.x & (CH - 1), pt = threadIdx.x >> 6;
    float a = 0.f;
#pragma unroll
    for (int s = pt; s < CH; s += PS) a += dTs[t * LF + s] * Af[t * LF + s];
    partr[pt][t] = a;
  }
  __syncthreads();
  if (threadIdx.x < CH) {
    const int t = threadIdx.x;
    float db = 0.f;
#pragma unroll
    for (int i = 0; i < PS; ++i) db += partc[i][t] + partr[i][t];
    if constexpr (LOG) db *= bs[t] * (1.f - bs[t]);
    if (t < n) dbeta[tk + t] = (E)db;
  }
}

// ---------------------------------------------------------------------------------------
// Backward, stage 3: per (chunk, head, 64 key channels).  The Gram slots
//   dk_s += sum_{t>s} dA_ts k_t e^{g_t-g_s} + sum_{t<s} dA_st k_t e^{g_s-g_t} + sum_{t>=s} dM_ts q_t e^{g_t-g_s}
//   dq_t += sum_{s<=t} dM_ts k_s e^{g_t-g_s}
// and d log alpha_t, the sum of every term whose decay factor spans token t:
//   sum_{s<t<=u} (dA_us k_u + dM_us q_u) k_s e^{g_u-g_s}
//   + sum_{u>=t} (q_u e^{g_u} dQhat_u + k_u e^{g_u} dKhat_u) + sum_{s<t} k_s e^{g_n-g_s} dKbar_s + gamma
// all as direct sums (no differences of running sums), so dalpha = d log alpha / alpha stays
// accurate for strongly decaying channels.  The 64 tokens form four 16-token blocks; wave b
// owns block b.  Pairs (u, s) in different blocks go through matrix-core products with
// reference tokens at block boundaries (factors <= 1); the pairs' contribution to d log alpha
// is assembled from those products' rows, block sums and block-pair totals.  Pairs inside a
// block use the block's first token as reference for dk and dq (matrix cores) and one lane
// per channel for their d log alpha terms; a block whose decay is too strong for that
// reference is summed exactly instead, one exponential per term.
// Eight waves: waves b and b + 4 share block b, each taking half of its column tiles in the
// matrix-core part, and in the channel layout half of the in-block pairs (by the later token)
// and half of the block's tokens for d log alpha.
// ---------------------------------------------------------------------------------------
template <typename E>
struct KdaGramLds {
  static constexpr int JW = 64, LDJ = JW + pad16<E>(), LDT = CH + pad16<E>(), LDF = JW + 1;
  static constexpr int GB = CH * LDF * 4, TJ = CH * LDJ * (int)sizeof(E), SQ = CH * LDT * (int)sizeof(E);
  static constexpr int ST = CH * LDF * 4;
  static constexpr int oG = 0, oK = GB, oQ = GB + TJ, oX = GB + 2 * TJ;
  // region X: dA | dM | Kend (48 rows) | Kf | Qf | Krf, later two float staging arrays and the
  // in-block pair sums one half of a block's waves hands to the other
  static constexpr int odA = oX, odM = oX + SQ, oKe = oX + 2 * SQ, oKf = oKe + 48 * LDJ * (int)sizeof(E);
  static constexpr int oQf = oKf + TJ, oKrf = oQf + TJ, endOps = oKrf + TJ;
  static constexpr int oS1 = oX, oS2 = oX + ST, oN4 = oX + 2 * ST;
  static constexpr int BYTES = cmax(endOps, oN4 + CH * JW * 4);
};

// LOG: alpha holds logits; dalpha is returned w.r.t. them: d log alpha * (-sigmoid(x)).
// EF: nothing erased: no dA slot (held at zero, its products skipped) and no dKhat term.
template <typename E, int D, bool LOG, bool EF, bool QKN>
__global__ __launch_bounds__(512) void k_bwd_kda_gram(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                      const E* __restrict__ alpha, E* __restrict__ dq,
                                                      E* __restrict__ dk, E* __restrict__ dalpha, Plan p) {
  GDR_POISON_ALL();
  using Ly = KdaGramLds<E>;
  constexpr int NT = 512, JW = Ly::JW, LDJ = Ly::LDJ, LDT = Ly::LDT, LDF = Ly::LDF, NC = JW / 16;
  constexpr int NCW = NC / 2;  // column tiles per wave
  __shared__ __align__(16) char smem[Ly::BYTES];
  __shared__ float c1s[3][JW], tota[4][JW], totc[4][JW];
  __shared__ int unsafe[4];
  // QKN (q/k normalisation): both channel halves run in this workgroup, one after the other;
  // the first half's dk~, dq~ wait in stK, stQ for the rows' x~ . dx~, whose parts (channel
  // half, column half of the waves) collect in pdk, pdq
  constexpr int NHZ = D / JW;
  static_assert(NHZ == 1 || NHZ == 2, "one or two channel halves");
  __shared__ __align__(16) E stK[NHZ > 1 ? CH * LDJ : 8], stQ[NHZ > 1 ? CH * LDJ : 8];
  __shared__ float pdk[NHZ][2][CH], pdq[NHZ][2][CH];
  float* Gs = reinterpret_cast<float*>(smem + Ly::oG);
  E* Ks = reinterpret_cast<E*>(smem + Ly::oK);
  E* Qs = reinterpret_cast<E*>(smem + Ly::oQ);
  E* dAs = reinterpret_cast<E*>(smem + Ly::odA);
  E* dMs = reinterpret_cast<E*>(smem + Ly::odM);
  E* Ke = reinterpret_cast<E*>(smem + Ly::oKe);
  E* Kf = reinterpret_cast<E*>(smem + Ly::oKf);
  E* Qf = reinterpret_cast<E*>(smem + Ly::oQf);
  E* Krf = reinterpret_cast<E*>(smem + Ly::oKrf);
  float* S1 = reinterpret_cast<float*>(smem + Ly::oS1);
  float* S2 = reinterpret_cast<float*>(smem + Ly::oS2);
  float* N4 = reinterpret_cast<float*>(smem + Ly::oN4);

  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int w = wave_id(), l = lane_id(), n = cp.n;
  const int b = w & 3;   // this wave's 16-token block
  const int hf = w >> 2; // this wave's half of the block's work
  constexpr int nhz = QKN ? NHZ : 1;
  // the halves as separate copies of the body (a loop kept registers live across them)
  static_for<0, nhz>([&](auto hzc) {
    constexpr int hz = decltype(hzc)::value;
    const int j0 = (QKN ? hz : (int)blockIdx.z) * JW;

    {
      RegTile<E, CH, JW, NT> rk, rq, ra;
      RegTile<E, CH, CH, NT> rda, rdm;
      float rnk[decltype(rk)::IT], rnq[decltype(rq)::IT];  // q/k normalisation: 1 / ||x|| of this thread's rows
      if constexpr (QKN) {
        load_row_factors(rk, p.Rn + u * 2 * CH + CH, rnk);
        load_row_factors(rq, p.Rn + u * 2 * CH, rnq);
      }
      ra.load(alpha + tk * D + j0, D, n);
      rk.load(k + tk * D + j0, D, n);
      rq.load(q + tk * D + j0, D, n);
      if constexpr (!EF) rda.load(reinterpret_cast<const E*>(p.kd_da) + u * CH * CH, CH, CH);
      rdm.load(reinterpret_cast<const E*>(p.kd_dm) + u * CH * CH, CH, CH);
      if (threadIdx.x < 4) unsafe[threadIdx.x] = 0;
      if constexpr (QKN) {  // this block's channels of the rows the preparation normalised
        scale_rows(rk, rnk);
        scale_rows(rq, rnq);
      }
      rk.store(Ks, LDJ);
      rq.store(Qs, LDJ);
      rdm.store(dMs, LDT);
      if constexpr (EF) {
        using RA = decltype(rda);
  #pragma unroll
        for (int it = 0; it < RA::IT; ++it) {
          if (RA::TOTAL % NT == 0 || threadIdx.x + it * NT < RA::TOTAL)
            *reinterpret_cast<typename RA::V*>(dAs + rda.row(it) * LDT + rda.col(it)) = typename RA::V{};
        }
      } else {
        rda.store(dAs, LDT);
      }
      kda_cumlog<E, JW, NT, LOG>(ra, n, Gs, LDF);
    }
    kda_flags<JW, NT>(Gs, LDF, unsafe);
    // Kend_s = k_s e^{g_{16(J+1)} - g_s} (s in block J < 3);  Kf_u, Qf_u = (k_u, q_u) e^{g_u - g_{16I}}
    // (u in block I);  Krf_s = k_s e^{g_{16I} - g_s} (zero in blocks summed exactly)
    {
      constexpr int VE = 16 / (int)sizeof(E);  // 16 bytes per step
      for (int idx = threadIdx.x; idx < CH * JW / VE; idx += NT) {
        const int s = idx / (JW / VE), jv = (idx % (JW / VE)) * VE, r0 = s & ~15;
        const bool uns = unsafe[s >> 4] != 0;
        const uint4 kv4 = *reinterpret_cast<const uint4*>(Ks + s * LDJ + jv);
        const uint4 qv4 = *reinterpret_cast<const uint4*>(Qs + s * LDJ + jv);
        const E* ke = reinterpret_cast<const E*>(&kv4);
        const E* qe = reinterpret_cast<const E*>(&qv4);
        uint4 ev, fv, qfv, rv;
        E* eo = reinterpret_cast<E*>(&ev);
        E* fo = reinterpret_cast<E*>(&fv);
        E* qo = reinterpret_cast<E*>(&qfv);
        E* ro = reinterpret_cast<E*>(&rv);
  #pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int j = jv + e;
          const float gs_ = Gs[s * LDF + j], g0 = Gs[r0 * LDF + j];
          const float kv = (float)ke[e];
          eo[e] = (E)(s < 48 ? kv * __expf(Gs[(min(r0 + 16, CH - 1)) * LDF + j] - gs_) : 0.f);
          const float f = __expf(gs_ - g0);
          fo[e] = (E)(kv * f);
          qo[e] = (E)((float)qe[e] * f);
          ro[e] = (E)(uns ? 0.f : kv * __expf(g0 - gs_));
        }
        if (s < 48) *reinterpret_cast<uint4*>(Ke + s * LDJ + jv) = ev;
        *reinterpret_cast<uint4*>(Kf + s * LDJ + jv) = fv;
        *reinterpret_cast<uint4*>(Qf + s * LDJ + jv) = qfv;
        *reinterpret_cast<uint4*>(Krf + s * LDJ + jv) = rv;
      }
    }
    __syncthreads();
    const bool exact = unsafe[b] != 0;  // wave-uniform

    // Loads of the last phases, issued now so that their latency is hidden: the partial
    // gradients from the earlier stages at this wave's matrix-core elements, and alpha and the
    // memory term at this lane's channel.
    const float* dqh = p.kd_dqh + u * CH * D;
    const float* dkh = p.kd_dkh + u * CH * D;
    const float* dkb = p.kd_dkb + u * CH * D;
    float lq[NCW][4], lk[NCW][4], lb[NCW][4], la[8];
  #pragma unroll
    for (int cc = 0; cc < NCW; ++cc) {
      const int o = frag_off<D>(b, j0 / 16 + hf * NCW + cc);
      const f32x4 x = *reinterpret_cast<const f32x4*>(dqh + o);
      const f32x4 y = EF ? zero4() : *reinterpret_cast<const f32x4*>(dkh + o);
      const f32x4 z = *reinterpret_cast<const f32x4*>(dkb + o);
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        lq[cc][r] = x[r];
        lk[cc][r] = y[r];
        lb[cc][r] = z[r];
      }
    }
  #pragma unroll
    for (int i = 0; i < 8; ++i) {  // this half's tokens of the block
      const int t = min(16 * b + 8 * hf + i, n - 1);
      la[i] = (float)alpha[(tk + t) * D + j0 + l];
    }
    const float gam_l = p.kd_gam[u * D + j0 + l];

    // ---- pairs inside block b, channel j0 + l: one lane per channel
    float n4[16], dkd[16], dqd[16];
  #pragma unroll
    for (int i = 0; i < 16; ++i) n4[i] = dkd[i] = dqd[i] = 0.f;
    {
      const E* dAb = dAs + 16 * b * LDT + 16 * b;
      const E* dMb = dMs + 16 * b * LDT + 16 * b;
      const float* gcol = Gs + 16 * b * LDF + l;
      const E* kcol = Ks + 16 * b * LDJ + l;
      const E* qcol = Qs + 16 * b * LDJ + l;
      if (!exact) {
        // d log alpha terms only: sum_{s<t<=u} c_us y_s with c_us = dA_us kF_u + dM_us qF_u,
        // y_s = k_s e^{g_b - g_s}, kF_u = k_u e^{g_u - g_b} (b = the block's first token)
        float kf[16], qf[16], y[16];
        const float g0 = gcol[0];
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float gi = gcol[i * LDF], kv = (float)kcol[i * LDJ];
          const float f = __expf(gi - g0);
          kf[i] = kv * f;
          qf[i] = (float)qcol[i * LDJ] * f;
          y[i] = kv * __expf(g0 - gi);
        }
        // later tokens uu = 1..10 in the first half, 11..15 in the second (55 and 65 pairs)
        const auto later = [&](auto uu_c) {
          constexpr int uu = decltype(uu_c)::value;
          float run = 0.f;
  #pragma unroll
          for (int s = 0; s < uu; ++s) {
            const float c = fmaf((float)dMb[uu * LDT + s], qf[uu], (float)dAb[uu * LDT + s] * kf[uu]);
            run = fmaf(c, y[s], run);
            n4[s + 1] += run;
          }
        };
        if (hf == 0) {
          static_for<1, 11>(later);
        } else {
          static_for<11, 16>(later);
        }
      } else if (hf == 0) {
        // exact: one exponential per pair; also the pairs' dk and dq
        float kk[16], gg[16];
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          kk[i] = (float)kcol[i * LDJ];
          gg[i] = gcol[i * LDF];
        }
  #pragma unroll 1
        for (int uu = 0; uu < 16; ++uu) {
          const float guu = gcol[uu * LDF], kuu = (float)kcol[uu * LDJ], quu = (float)qcol[uu * LDJ];
          float run = 0.f, ak = 0.f, aq = 0.f;
  #pragma unroll
          for (int s = 0; s < 16; ++s) {
            const bool m = s < uu;
            const float e = m ? __expf(guu - gg[s]) : 0.f;
            const float da = m ? (float)dAb[uu * LDT + s] : 0.f, dm = m ? (float)dMb[uu * LDT + s] : 0.f;
            const float ce = (da * kuu + dm * quu) * e;
            dkd[s] += ce;
            const float ke = kk[s] * e;
            ak += da * ke;
            aq += dm * ke;
            run += ce * kk[s];
            if (s < 15 && m) n4[s + 1] += run;
          }
          const float dmd = (float)dMb[uu * LDT + uu];
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (i == uu) {
              dkd[i] += ak + dmd * quu;
              dqd[i] += aq + dmd * kuu;
            }
          }
        }
      }
    }

    // ---- matrix-core part (waves b and b + 4 own the output rows of block b, half of the column
    // tiles each).  Accumulated per element:
    // dkacc, dqacc: every dk / dq term from these products;  y2 = k * (dk lower, other blocks)
    // + q * (dq, other blocks): block-suffix terms;  x3 = k * (dk upper, other blocks): block-prefix terms.
    f32x4 dkacc[NCW], dqacc[NCW], y2[NCW], x3[NCW];
  #pragma unroll
    for (int cc = 0; cc < NCW; ++cc) dkacc[cc] = dqacc[cc] = y2[cc] = x3[cc] = zero4();
  #pragma unroll
    for (int cc = 0; cc < NCW; ++cc) {
      const int c = hf * NCW + cc;
      const int j = acc_col(16 * c);
      float kv[4], qv[4], gv[4];
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int uu = acc_row(16 * b, r);
        kv[r] = (float)Ks[uu * LDJ + j];
        qv[r] = (float)Qs[uu * LDJ + j];
        gv[r] = Gs[uu * LDF + j];
      }
  #pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J < b) {  // lower: u in block b, s in block J
          f32x4 pa = zero4();
          if constexpr (!EF) pa = mma16<E>(zero4(), rowk(dAs, LDT), 16 * b, colk(Ke, LDJ), 16 * c, 16 * J);
          const f32x4 pm = mma16<E>(zero4(), rowk(dMs, LDT), 16 * b, colk(Ke, LDJ), 16 * c, 16 * J);
          const float gref = Gs[16 * (J + 1) * LDF + j];
          float ps = 0.f;
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float f = __expf(gv[r] - gref);
            const float a = f * pa[r], m = f * pm[r];
            dkacc[cc][r] += a;
            dqacc[cc][r] += m;
            const float pr = kv[r] * a + qv[r] * m;
            y2[cc][r] += pr;
            ps += pr;
          }
          // the pair (b, J)'s total, needed by the blocks strictly between J and b: pairs (2, 0),
          // (3, 0) and (3, 1) into c1s[0..2] (no block lies between 2 and 3)
          if ((b == 2 && J == 0) || (b == 3 && J < 2)) {
            ps += __shfl_xor(ps, 16, 64);
            ps += __shfl_xor(ps, 32, 64);
            if (l < 16) c1s[(b == 2) ? 0 : 1 + J][j] = ps;
          }
        }
      }
  #pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I > b) {  // upper: s in block b, u in block I
          f32x4 ua = zero4();
          if constexpr (!EF) ua = mma16<E>(zero4(), colk(dAs, LDT), 16 * b, colk(Kf, LDJ), 16 * c, 16 * I);
          ua = mma16<E>(ua, colk(dMs, LDT), 16 * b, colk(Qf, LDJ), 16 * c, 16 * I);
          const float gref = Gs[16 * I * LDF + j];
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = __expf(gref - gv[r]) * ua[r];
            dkacc[cc][r] += x;
            x3[cc][r] += kv[r] * x;
          }
        }
      }
      if (!exact) {  // pairs inside block b, first token of the block as reference
        f32x4 pa = zero4(), ua = zero4();
        if constexpr (!EF) {
          pa = mma16<E>(zero4(), rowk(dAs, LDT), 16 * b, colk(Krf, LDJ), 16 * c, 16 * b);
          ua = mma16<E>(zero4(), colk(dAs, LDT), 16 * b, colk(Kf, LDJ), 16 * c, 16 * b);
        }
        const f32x4 pm = mma16<E>(zero4(), rowk(dMs, LDT), 16 * b, colk(Krf, LDJ), 16 * c, 16 * b);
        ua = mma16<E>(ua, colk(dMs, LDT), 16 * b, colk(Qf, LDJ), 16 * c, 16 * b);
        const float g0 = Gs[16 * b * LDF + j];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float f = __expf(gv[r] - g0), rf = __expf(g0 - gv[r]);
          dkacc[cc][r] += f * pa[r] + rf * ua[r];
          dqacc[cc][r] += f * pm[r];
        }
      }
    }
    __syncthreads();  // region X becomes the staging area
    if (exact && hf == 0) {
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        S1[(16 * b + i) * LDF + l] = dkd[i];
        S2[(16 * b + i) * LDF + l] = dqd[i];
      }
    }
    __syncthreads();

    // ---- dq, dk, and the per-row terms of d log alpha (matrix-core layout)
    float pa_[NCW], pc_[NCW];
    float xk4[4] = {0.f, 0.f, 0.f, 0.f}, xq4[4] = {0.f, 0.f, 0.f, 0.f};  // k~ . dk~, q~ . dq~ (QKN)
  #pragma unroll
    for (int cc = 0; cc < NCW; ++cc) {
      const int c = hf * NCW + cc;
      const int j = acc_col(16 * c);
      const float gn = Gs[(CH - 1) * LDF + j];
      float sa = 0.f, sc = 0.f;
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int uu = acc_row(16 * b, r);
        const float g = Gs[uu * LDF + j], eg = __expf(g), egb = __expf(gn - g);
        const float kv = (float)Ks[uu * LDJ + j], qv = (float)Qs[uu * LDJ + j];
        const float xq = eg * lq[cc][r], xk = eg * lk[cc][r], xb = egb * lb[cc][r];
        float dkv = dkacc[cc][r] + xk + xb, dqv = dqacc[cc][r] + xq;
        if (exact) {
          dkv += S1[uu * LDF + j];
          dqv += S2[uu * LDF + j];
        }
        // dk, dq replace this lane's own elements of K and Q (read just above; rows of block b
        // are read by this wave only) and go out as whole rows below
        Ks[uu * LDJ + j] = (E)dkv;
        Qs[uu * LDJ + j] = (E)dqv;
        if constexpr (QKN) {
          xk4[r] += kv * dkv;
          xq4[r] += qv * dqv;
        }
        const float a = qv * xq + kv * xk, bt = kv * xb;
        y2[cc][r] += a;
        x3[cc][r] += bt;
        sa += a;
        sc += bt;
      }
      sa += __shfl_xor(sa, 16, 64);
      sa += __shfl_xor(sa, 32, 64);
      sc += __shfl_xor(sc, 16, 64);
      sc += __shfl_xor(sc, 32, 64);
      pa_[cc] = sa;
      pc_[cc] = sc;
    }
    if constexpr (QKN) {  // this wave's part of each row's dot: its columns are the 16 lanes of a row group
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = xk4[r], c = xq4[r];
  #pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          a += __shfl_xor(a, off, 64);
          c += __shfl_xor(c, off, 64);
        }
        if (lrow() == 0) {
          pdk[hz][hf][acc_row(16 * b, r)] = a;
          pdq[hz][hf][acc_row(16 * b, r)] = c;
        }
      }
    }
    __syncthreads();
    if constexpr (!QKN) {
      s2g_rows<E, CH, JW, NT>(dk + tk * D + j0, D, Ks, LDJ, n);
      s2g_rows<E, CH, JW, NT>(dq + tk * D + j0, D, Qs, LDJ, n);
    } else if constexpr (hz + 1 < nhz) {  // kept until the other half's dots are in
      constexpr int VE = 16 / (int)sizeof(E);
      for (int idx = threadIdx.x; idx < CH * JW / VE; idx += NT) {
        const int t = idx / (JW / VE), c0 = (idx % (JW / VE)) * VE;
        *reinterpret_cast<uint4*>(stK + t * LDJ + c0) = *reinterpret_cast<const uint4*>(Ks + t * LDJ + c0);
        *reinterpret_cast<uint4*>(stQ + t * LDJ + c0) = *reinterpret_cast<const uint4*>(Qs + t * LDJ + c0);
      }
    }
  #pragma unroll
    for (int cc = 0; cc < NCW; ++cc) {
      const int c = hf * NCW + cc;
      store4_n(S1, LDF, 16 * b, 16 * c, y2[cc]);
      store4_n(S2, LDF, 16 * b, 16 * c, x3[cc]);
      if (l < 16) {
        tota[b][16 * c + l] = pa_[cc];
        totc[b][16 * c + l] = pc_[cc];
      }
    }
    // the in-block pair sums at the other half's tokens
  #pragma unroll
    for (int i = 0; i < 8; ++i) N4[(16 * b + 8 * (1 - hf) + i) * JW + l] = hf ? n4[i] : n4[8 + i];
    __syncthreads();

    // ---- d log alpha, channel layout
    {
      float cross = gam_l;
  #pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        if (bb > b) cross += tota[bb][l];
        if (bb < b) cross += totc[bb][l];
      }
      if (b == 1) cross += c1s[0][l] + c1s[1][l];
      if (b == 2) cross += c1s[1][l] + c1s[2][l];
      // this half's tokens t0 .. t0 + 7: suffix sums of S1 from the block's end, prefix sums of S2
      // from its start, in the same order as over the whole block
      const int t0 = 16 * b + 8 * hf;
      float suf[8];
      float run = 0.f;
      if (hf == 0) {
  #pragma unroll
        for (int i = 15; i >= 8; --i) run += S1[(16 * b + i) * LDF + l];
      }
  #pragma unroll
      for (int i = 7; i >= 0; --i) {
        run += S1[(t0 + i) * LDF + l];
        suf[i] = run;
      }
      run = 0.f;
      if (hf == 1) {
  #pragma unroll
        for (int i = 0; i < 8; ++i) run += S2[(16 * b + i) * LDF + l];
      }
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + i;
        const float dla = ((hf ? n4[8 + i] : n4[i]) + N4[t * JW + l]) + suf[i] + run + cross;
        run += S2[t * LDF + l];
        if (t < n) {
          if constexpr (LOG) dalpha[(tk + t) * D + j0 + l] = (E)(-dla * gate_sigmoid(la[i]));
          else dalpha[(tk + t) * D + j0 + l] = (E)(dla / la[i]);
        }
      }
    }
    __syncthreads();  // the next channel half reuses the LDS regions
  });
  if constexpr (QKN) {  // dq, dk w.r.t. the raw rows: dx = (dx~ - x~ (x~ . dx~)) / ||x||, both halves
    for (int hz = 0; hz < nhz; ++hz) {
      const int j0 = hz * JW;
      const E* sk = hz + 1 < nhz ? stK : Ks;
      const E* sq = hz + 1 < nhz ? stQ : Qs;
      using RT = RegTile<E, CH, JW, NT>;
      RT xk, xq;  // this half of the normalised rows, formed as the preparation formed them
      float fk[RT::IT], fq[RT::IT];
      load_row_factors(xk, p.Rn + u * 2 * CH + CH, fk);
      load_row_factors(xq, p.Rn + u * 2 * CH, fq);
      xk.load(k + tk * D + j0, D, n);
      xq.load(q + tk * D + j0, D, n);
      scale_rows(xk, fk);
      scale_rows(xq, fq);
#pragma unroll
      for (int it = 0; it < RT::IT; ++it) {
        const int t = xk.row(it), c0 = xk.col(it);
        if ((RT::TOTAL % NT != 0 && threadIdx.x + it * NT >= RT::TOTAL) || t >= n) continue;
        float dk_ = 0.f, dq_ = 0.f;
#pragma unroll
        for (int z = 0; z < NHZ; ++z) {
          dk_ += pdk[z][0][t] + pdk[z][1][t];
          dq_ += pdq[z][0][t] + pdq[z][1][t];
        }
        typename RT::V ok, oq;
        E* oke = reinterpret_cast<E*>(&ok);
        E* oqe = reinterpret_cast<E*>(&oq);
        const typename RT::V gk = *reinterpret_cast<const typename RT::V*>(sk + t * LDJ + c0);
        const typename RT::V gq = *reinterpret_cast<const typename RT::V*>(sq + t * LDJ + c0);
        const E* gke = reinterpret_cast<const E*>(&gk);
        const E* gqe = reinterpret_cast<const E*>(&gq);
#pragma unroll
        for (int x = 0; x < RT::VE; ++x) {
          oke[x] = (E)(((float)gke[x] - dk_ * (float)xk.elem(it, x)) * fk[it]);
          oqe[x] = (E)(((float)gqe[x] - dq_ * (float)xq.elem(it, x)) * fq[it]);
        }
        *reinterpret_cast<typename RT::V*>(dk + (tk + t) * D + j0 + c0) = ok;
        *reinterpret_cast<typename RT::V*>(dq + (tk + t) * D + j0 + c0) = oq;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Erase-free backward, stage 2: with R = U = diag(beta) V the solve side reduces to
//   dv_t = beta_t dR_t,  dbeta_t = v_t . dR_t   (beta absent: dv = dR, no dbeta).
// One workgroup per (chunk, head); a row of the tile is VPR adjacent lanes.
// LOG: beta is a logit; dbeta is returned w.r.t. it (times beta (1 - beta)).
// ---------------------------------------------------------------------------------------
template <typename E, int D, bool LOG>
__global__ __launch_bounds__(256) void k_bwd_gla_wv(Geo geo, const E* __restrict__ v, const E* __restrict__ beta,
                                                    const E* __restrict__ dRg, E* __restrict__ dv,
                                                    E* __restrict__ dbeta) {
  GDR_POISON_ALL();
  constexpr int NT = 256;
  using RT = RegTile<E, CH, D, NT>;
  static_assert(RT::VB == 16 && RT::TOTAL % NT == 0, "whole 16-byte rows per lane group");
  const int gc = blockIdx.x, h = blockIdx.y;
  const ChunkPos cp = chunk_pos(geo, gc);
  const long u = (long)gc * geo.H + h;
  const long tk = tok_index(geo, cp.b, h, cp.t0);
  const int n = cp.n;
  RT rv, rd;
  rv.load(v + tk * D, D, n);
  rd.load(dRg + u * CH * D, D, CH);
#pragma unroll
  for (int it = 0; it < RT::IT; ++it) {
    const int t = rv.row(it), c = rv.col(it);
    float b = 1.f;
    if (beta) {
      b = (float)beta[tk + min(t, n - 1)];
      if constexpr (LOG) b = gate_sigmoid(b);
    }
    const E* de = reinterpret_cast<const E*>(&rd.v[it]);
    typename RT::V ov;
    E* oe = reinterpret_cast<E*>(&ov);
    float dot = 0.f;
#pragma unroll
    for (int x = 0; x < RT::VE; ++x) {
      const float d = (float)de[x];
      dot += (float)rv.elem(it, x) * d;
      oe[x] = (E)(b * d);
    }
    if (t < n) *reinterpret_cast<typename RT::V*>(dv + (tk + t) * D + c) = ov;
    if (dbeta) {
      dot = group_sum_dpp<RT::VPR>(dot);
      if (threadIdx.x % RT::VPR == 0 && t < n) dbeta[tk + t] = (E)(LOG ? dot * b * (1.f - b) : dot);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
template <typename E, int D>
hipError_t launch_fwd_prep_kda(const Plan& p, const gdr_inputs& in, hipStream_t st) {
  const bool ef = p.variant == GDR_GLA;
  TraceScope ts_(ef ? "fwd_prep_gla" : "fwd_prep_kda", st);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(p.geo.total_chunks, p.geo.H), dim3(512), 0, st, p.geo, (const E*)in.q,
                       (const E*)in.k, (const E*)in.v, (const E*)in.beta, (const E*)in.alpha, (E*)p.X, (E*)p.Ub,
                       (E*)p.M, (E*)p.Kb, (E*)p.Qh, p.Gn, p.Li, p.A1, p.qkn ? p.Rn : nullptr);
  };
  if (ef) {
    if (p.gates) go(k_fwd_prep_kda<E, D, true, true>);
    else go(k_fwd_prep_kda<E, D, false, true>);
  } else {
    if (p.gates) go(k_fwd_prep_kda<E, D, true, false>);
    else go(k_fwd_prep_kda<E, D, false, false>);
  }
  return hipGetLastError();
}
template hipError_t launch_fwd_prep_kda<bf16, 128>(const Plan&, const gdr_inputs&, hipStream_t);
template hipError_t launch_fwd_prep_kda<bf16, 64>(const Plan&, const gdr_inputs&, hipStream_t);
template hipError_t launch_fwd_prep_kda<float, 64>(const Plan&, const gdr_inputs&, hipStream_t);

template <typename E, int D>
hipError_t launch_bwd_kda(const Plan& p, const gdr_inputs& in, const void* dO, const gdr_grads& gr, hipStream_t st) {
  const dim3 grid(p.geo.total_chunks, p.geo.H);
  if (p.variant == GDR_GLA) {
    {
      TraceScope ts_("bwd_gla_state", st);
      hipLaunchKernelGGL((k_bwd_kda_state<E, D, true>), grid, dim3(512), 0, st, p.geo, (const E*)dO,
                         (const float*)p.Gn, (const E*)p.Hs, (const E*)p.R, (const E*)p.dHs, (const E*)p.dR, p);
    }
    {
      TraceScope ts_("bwd_gla_wv", st);
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, p.geo, (const E*)in.v, (const E*)in.beta, (const E*)p.dR,
                           (E*)gr.dv, (E*)gr.dbeta);
      };
      if (p.gates) go(k_bwd_gla_wv<E, D, true>);
      else go(k_bwd_gla_wv<E, D, false>);
    }
    {
      TraceScope ts_("bwd_gla_gram", st);
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(p.geo.total_chunks, p.geo.H, p.qkn ? 1 : D / 64), dim3(512), 0, st, p.geo,
                           (const E*)in.q, (const E*)in.k, (const E*)in.alpha, (E*)gr.dq, (E*)gr.dk,
                           (E*)gr.dalpha, p);
      };
      if (p.qkn) {
        if (p.gates) go(k_bwd_kda_gram<E, D, true, true, true>);
        else go(k_bwd_kda_gram<E, D, false, true, true>);
      } else {
        if (p.gates) go(k_bwd_kda_gram<E, D, true, true, false>);
        else go(k_bwd_kda_gram<E, D, false, true, false>);
      }
    }
    return hipGetLastError();
  }
  {
    TraceScope ts_("bwd_kda_state", st);
    hipLaunchKernelGGL((k_bwd_kda_state<E, D, false>), grid, dim3(512), 0, st, p.geo, (const E*)dO,
                       (const float*)p.Gn, (const E*)p.Hs, (const E*)p.R, (const E*)p.dHs, (const E*)p.dR, p);
  }
  {
    TraceScope ts_("bwd_kda_wy", st);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, p.geo, (const E*)in.k, (const E*)in.v, (const E*)in.beta,
                         (const E*)in.alpha, (const E*)p.dR, (E*)gr.dv, (E*)gr.dbeta, p);
    };
    if (p.gates) go(k_bwd_kda_wy<E, D, true>);
    else go(k_bwd_kda_wy<E, D, false>);
  }
  {
    TraceScope ts_("bwd_kda_gram", st);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(p.geo.total_chunks, p.geo.H, p.qkn ? 1 : D / 64), dim3(512), 0, st, p.geo, (const E*)in.q,
                         (const E*)in.k, (const E*)in.alpha, (E*)gr.dq, (E*)gr.dk, (E*)gr.dalpha, p);
    };
    if (p.qkn) {
      if (p.gates) go(k_bwd_kda_gram<E, D, true, false, true>);
      else go(k_bwd_kda_gram<E, D, false, false, true>);
    } else {
      if (p.gates) go(k_bwd_kda_gram<E, D, true, false, false>);
      else go(k_bwd_kda_gram<E, D, false, false, false>);
    }
  }
  return hipGetLastError();
}
template hipError_t launch_bwd_kda<bf16, 128>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);
template hipError_t launch_bwd_kda<bf16, 64>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);
template hipError_t launch_bwd_kda<float, 64>(const Plan&, const gdr_inputs&, const void*, const gdr_grads&, hipStream_t);

}  // namespace gdr
