// The gradient of the q/k L2-normalisation (queries and keys scaled to unit length per token,
// y = x / ||x||_2 over the head dimension, a zero row left zero) for the variants whose backward
// produces dq, dk w.r.t. the normalised rows (Kimi Delta Attention and the erase-free variant,
// whose Gram stage holds half of a row's channels; the kernels apply the normalisation itself):
//   dx = (dy - y (y . dy)) / ||x||.
// Unit-length keys keep the delta rule's rank-1 factor I - beta k k^T with eigenvalue 1 - beta.
// A memory-bound elementwise pass over [rows, d] token rows, 16-byte vectors, float32 arithmetic.
#include <algorithm>

#include "launch.hpp"

namespace gdr {

// A row of D elements is spread over LPR lanes holding one 16-byte vector each (D * esz / 16
// lanes: 16 for 128 bf16 or 64 float32, 8 for 64 bf16), so a wave covers 64 / LPR rows per
// step; the grid strides over the rows.  Norms and dot products are reduced across the row's
// lanes with exchanges inside the lane group.
template <typename E, int D>
struct RowVec {
  static constexpr int VE = 16 / (int)sizeof(E), LPR = D / VE;
  static_assert(64 % LPR == 0, "whole rows per wave");
  uint4 raw;
  __device__ __forceinline__ void load(const E* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float at(int i) const { return (float)reinterpret_cast<const E*>(&raw)[i]; }
};
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
template <typename E, int VE>
__device__ __forceinline__ void store_vec(E* p, const float* v) {
  uint4 raw;
  E* e = reinterpret_cast<E*>(&raw);
#pragma unroll
  for (int i = 0; i < VE; ++i) e[i] = (E)v[i];
  *reinterpret_cast<uint4*>(p) = raw;
}

// dx = (dy - y (y . dy)) / ||x|| in place over dy, y recomputed from x.
template <typename E, int D>
__global__ __launch_bounds__(256) void k_l2norm_grad_rows(const E* __restrict__ x, E* __restrict__ dxy, long rows) {
  GDR_POISON_ALL();
  using RV = RowVec<E, D>;
  constexpr int VE = RV::VE, LPR = RV::LPR;
  const long g0 = ((long)blockIdx.x * 256 + threadIdx.x) / LPR, stride = (long)gridDim.x * 256 / LPR;
  const int c = (threadIdx.x % LPR) * VE;
  for (long row = g0; row < rows; row += stride) {
    RV a, b;
    a.load(x + row * D + c);
    b.load(dxy + row * D + c);
    float v[VE], g[VE], ss = 0.f, yg = 0.f;
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      v[i] = a.at(i);
      g[i] = b.at(i);
      ss += v[i] * v[i];
      yg += v[i] * g[i];
    }
    ss = group_sum<LPR>(ss);
    yg = group_sum<LPR>(yg);
    const float rn = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
    const float ygn = yg * rn * rn;  // y . dy with y = x rn
#pragma unroll
    for (int i = 0; i < VE; ++i) g[i] = (g[i] - v[i] * ygn) * rn;
    store_vec<E, VE>(dxy + row * D + c, g);
  }
}

hipError_t run_l2norm_grad(int dtype, int D, const void* x, void* dxy, long rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  TraceScope ts_("l2norm_grad", st);
  // 16-byte vectors: D * esz / 16 threads per row; at most eight workgroups per CU, then stride
  const long threads = rows * ((long)D * (dtype == GDR_BF16 ? 2 : 4) / 16);
  const dim3 grid((unsigned)std::min<long>((threads + 255) / 256, 2048));
  auto go = [&](auto kern, auto* px, auto* py) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, px, py, rows); };
  if (dtype == GDR_BF16) {
    const bf16* px = static_cast<const bf16*>(x);
    bf16* py = static_cast<bf16*>(dxy);
    if (D == 128) go(k_l2norm_grad_rows<bf16, 128>, px, py);
    else go(k_l2norm_grad_rows<bf16, 64>, px, py);
  } else {
    go(k_l2norm_grad_rows<float, 64>, static_cast<const float*>(x), static_cast<float*>(dxy));
  }
  return hipGetLastError();
}

}  // namespace gdr
