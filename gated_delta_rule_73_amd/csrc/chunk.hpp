// Chunk-local pieces shared by the forward and backward kernels.
#pragma once

#include "common.hpp"

namespace gdr {

enum Var { VAR_DELTANET = 0, VAR_GATED = 1, VAR_KDA = 2, VAR_GDN2 = 3 };

// Li = L^{-1} for a unit lower-triangular 64x64 float matrix L (only entries strictly below
// the diagonal are read).  Blocked in 16x16 tiles: each diagonal tile is inverted by
// right-looking substitution (one lane per column), then the tiles below the diagonal are
// filled in order of their distance from it, X_ij = -inv(L_ii) * sum_{j<=m<i} L_im X_mj,
// with float32 matrix-core products.  scratch: 4*256 floats.  Needs >= 256 threads; ends
// with a block barrier.  Li's tiles above the diagonal are set to zero.
template <int NT>
__device__ void solve_unit_lower64(const float* L, int ldl, float* Li, int ldi, float* scratch) {
  static_assert(NT >= 256, "solve needs four waves");
  const int w = wave_id(), l = lane_id();
  if (w < 4 && l < 16) {
    const int c = l, o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
      for (int r = kk + 1; r < 16; ++r) x[r] = fmaf(-L[(o + r) * ldl + o + kk], x[kk], x[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Li[(o + r) * ldi + o + c] = x[r];
  }
  for (int idx = threadIdx.x; idx < 64 * 64; idx += NT) {
    const int r = idx >> 6, c = idx & 63;
    if ((c >> 4) > (r >> 4)) Li[r * ldi + c] = 0.f;
  }
  __syncthreads();
  for (int dist = 1; dist < 4; ++dist) {
    const bool act = w < 4 - dist;
    const int j = w, i = w + dist;
    if (act) {
      f32x4 acc = zero4();
      for (int m = j; m < i; ++m)
        acc = mma_k<float, 16>(acc, rowk(L + (16 * i) * ldl + 16 * m, ldl), 0,
                               colk(Li + (16 * m) * ldi + 16 * j, ldi), 0);
      store4_n(scratch + w * 256, 16, 0, 0, acc);
    }
    __syncthreads();
    if (act) {
      const f32x4 acc = mma_k<float, 16>(zero4(), rowk(Li + (16 * i) * ldi + 16 * i, ldi), 0,
                                         colk(scratch + w * 256, 16), 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Li[(16 * i + acc_row(0, r)) * ldi + 16 * j + acc_col(0)] = -acc[r];
    }
    __syncthreads();
  }
}

// T^T as a matrix-core A operand, read from L^{-1}: element (m = s, k = t) = Linv[t][s] beta_s.
struct TtView {
  const float* li;
  int ld;
  const float* beta;
  __device__ __forceinline__ float at(int m, int k) const { return li[k * ld + m] * beta[m]; }
};
template <typename E>
__device__ __forceinline__ typename MMA<E>::frag frag(const TtView& v, int idx0, int k0) {
  constexpr int KPL = MMA<E>::KPL;
  const int m = idx0 + lrow(), kk = k0 + KPL * lgrp();
  if constexpr (KPL == 1) {
    return (E)v.at(m, kk);
  } else {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)v.at(m, kk + e);
    return r;
  }
}

// Map a lower-triangle tile index (0..9) of a 4x4 tile grid to (row tile, column tile).
__device__ __forceinline__ void tri_tile(int jj, int& mt, int& nt) {
  mt = (jj >= 1) + (jj >= 3) + (jj >= 6);
  nt = jj - mt * (mt + 1) / 2;
}

}  // namespace gdr
