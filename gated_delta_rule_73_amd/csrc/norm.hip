// q/k L2-normalisation around the chunked operator: queries and keys scaled to unit length per
// token (y = x / ||x||_2 over the head dimension, a zero row left zero) before the forward and
// backward, and the gradient carried back through the scaling after the backward,
//   dx = (dy - y (y . dy)) / ||x||.
// Unit-length keys keep the delta rule's rank-1 factor I - beta k k^T with eigenvalue 1 - beta.
// Memory-bound elementwise passes over [rows, d] token rows, one wave per row (d <= 128: one
// or two elements per lane), float32 arithmetic.
#include "launch.hpp"

namespace gdr {

template <typename E>
__device__ __forceinline__ float ld(const E* p) { return (float)*p; }

// y = x / ||x|| per row of d (d = 64 or 128).
template <typename E, int D>
__global__ __launch_bounds__(256) void k_l2norm_rows(const E* __restrict__ x, E* __restrict__ y, long rows) {
  constexpr int PL = D / 64;  // elements per lane
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = threadIdx.x & 63;
  const E* xr = x + row * D;
  float v[PL], ss = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    v[i] = ld(xr + l + 64 * i);
    ss += v[i] * v[i];
  }
  ss = wave_sum(ss);
  const float rn = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) y[row * D + l + 64 * i] = (E)(v[i] * rn);
}

// dx = (dy - y (y . dy)) / ||x|| in place over dy, y recomputed from x.
template <typename E, int D>
__global__ __launch_bounds__(256) void k_l2norm_grad_rows(const E* __restrict__ x, E* __restrict__ dxy, long rows) {
  constexpr int PL = D / 64;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = threadIdx.x & 63;
  float v[PL], g[PL], ss = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    v[i] = ld(x + row * D + l + 64 * i);
    g[i] = ld(dxy + row * D + l + 64 * i);
    ss += v[i] * v[i];
  }
  ss = wave_sum(ss);
  const float rn = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  float yg = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) yg += v[i] * rn * g[i];
  yg = wave_sum(yg);
#pragma unroll
  for (int i = 0; i < PL; ++i) dxy[row * D + l + 64 * i] = (E)((g[i] - v[i] * rn * yg) * rn);
}

hipError_t run_l2norm(int dtype, int D, const void* x, void* y, long rows, bool grad, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  TraceScope ts_(grad ? "l2norm_grad" : "l2norm", st);
  const dim3 grid((unsigned)((rows + 3) / 4));
  auto go = [&](auto fwd, auto bwd, auto* px, auto* py) {
    if (grad) hipLaunchKernelGGL(bwd, grid, dim3(256), 0, st, px, py, rows);
    else hipLaunchKernelGGL(fwd, grid, dim3(256), 0, st, px, py, rows);
  };
  if (dtype == GDR_BF16) {
    const bf16* px = static_cast<const bf16*>(x);
    bf16* py = static_cast<bf16*>(y);
    if (D == 128) go(k_l2norm_rows<bf16, 128>, k_l2norm_grad_rows<bf16, 128>, px, py);
    else go(k_l2norm_rows<bf16, 64>, k_l2norm_grad_rows<bf16, 64>, px, py);
  } else {
    const float* px = static_cast<const float*>(x);
    float* py = static_cast<float*>(y);
    go(k_l2norm_rows<float, 64>, k_l2norm_grad_rows<float, 64>, px, py);
  }
  return hipGetLastError();
}

}  // namespace gdr
