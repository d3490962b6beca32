// Chunk-local pieces shared by the forward and backward kernels.
#pragma once

#include "common.hpp"

namespace gdr {

// VAR_GDN2L: Gated DeltaNet-2 with its gates (beta, alpha, erase, write) given as logits.
// VAR_GLA: the erase-free memory with a decay per key channel, W <- W diag(alpha) + beta v k^T:
// Kimi Delta Attention's chunk form with nothing erased (A = 0, L = I, X = 0, R = U = beta V).
enum Var { VAR_DELTANET = 0, VAR_GATED = 1, VAR_KDA = 2, VAR_GDN2 = 3, VAR_GDN2L = 4, VAR_GLA = 5 };

// Li = L^{-1} for a unit lower-triangular 64x64 float matrix L (only entries strictly below
// the diagonal are read).  Blocked:
//   1. each 16x16 diagonal tile is inverted by forward substitution, one lane per column,
//      rows of L read as 16-byte vectors;
//   2. inside each 32x32 diagonal half, X_10 = -inv(L_11) L_10 inv(L_00) on 16x16 tiles
//      (one wave per half; the intermediate stays in that wave's scratch);
//   3. the lower-left 32x32 block, X = -inv(L_hh) L_hl inv(L_ll), with all four waves.
// Float32 matrix-core products throughout.  scratch: 4*256 floats.  Needs >= 256 threads;
// ends with a block barrier.  Li's entries above the diagonal are set to zero.  ldl, ldi must
// be multiples of 4 (16-byte rows).
template <int NT>
__device__ __forceinline__ void solve_unit_lower64(const float* L, int ldl, float* Li, int ldi, float* scratch) {
  static_assert(NT >= 256, "solve needs four waves");
  const int w = wave_id(), l = lane_id();
  if (w < 4 && l < 16) {
    const int c = l, o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // x_r = [r == c] - sum_{k<r} L_rk x_k
      float row[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(L + (o + r) * ldl + o + 4 * q);
        row[4 * q] = v.x; row[4 * q + 1] = v.y; row[4 * q + 2] = v.z; row[4 * q + 3] = v.w;
      }
      float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < r; ++k) acc = fmaf(-row[k], x[k], acc);
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Li[(o + r) * ldi + o + c] = x[r];
  }
  static_assert(64 * 16 % NT == 0, "whole 16-byte vectors per thread");
#pragma unroll
  for (int i = 0; i < 64 * 16 / NT; ++i) {  // four columns at a time
    const int idx = threadIdx.x + i * NT, r = idx >> 4, c0 = (idx & 15) * 4;
    if ((c0 >> 4) > (r >> 4)) *reinterpret_cast<float4*>(Li + r * ldi + c0) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  if (w < 2) {  // 16x16 merge inside half w: rows 32w+16.., columns 32w..
    const int a = 32 * w;
    const f32x4 y = mma_k<float, 16>(zero4(), rowk(L + (a + 16) * ldl + a, ldl), 0, colk(Li + a * ldi + a, ldi), 0);
    float* sc = scratch + w * 256;
    store4_n(sc, 16, 0, 0, y);
    const f32x4 xv = mma_k<float, 16>(zero4(), rowk(Li + (a + 16) * ldi + a + 16, ldi), 0, colk(sc, 16), 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) Li[(a + 16 + acc_row(0, r)) * ldi + a + acc_col(0)] = -xv[r];
  }
  __syncthreads();
  if (w < 4) {  // Y = L_hl inv(L_ll): rows 32.., columns 0..31; one 16x16 tile per wave
    const int mt = w >> 1, nt = w & 1;
    const f32x4 y = mma_k<float, 32>(zero4(), rowk(L + 32 * ldl, ldl), 16 * mt, colk(Li, ldi), 16 * nt);
    store4_n(scratch, 32, 16 * mt, 16 * nt, y);
  }
  __syncthreads();
  if (w < 4) {  // X = -inv(L_hh) Y
    const int mt = w >> 1, nt = w & 1;
    const f32x4 xv = mma_k<float, 32>(zero4(), rowk(Li + 32 * ldi + 32, ldi), 16 * mt, colk(scratch, 32), 16 * nt);
#pragma unroll
    for (int r = 0; r < 4; ++r) Li[(32 + acc_row(16 * mt, r)) * ldi + acc_col(16 * nt)] = -xv[r];
  }
  __syncthreads();
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
