// Segment combine for segmented scans: the start memory of every segment of a sequence.
//
// Per memory, segment s's map is W_end = W_start P_s + H_s (forward, segments in order) or
// dW_start = dW_end Q_s + G_s (backward, segments in reverse order), written by the scans'
// mode 1 as [additive part, linear part] in float32.  Starting from h0 (or dht, or zero), the
// kernel walks the segments, records each segment's start and applies its map with float32
// matrix-core products.  One workgroup per (memory, value-row tile); the tiles of a memory are
// independent (row i of W P depends only on row i of W).
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

template <int D, int BV>
__global__ __launch_bounds__(256) void k_seg_combine(Geo geo, ScanSeg sg, const float* __restrict__ init,
                                                     float* __restrict__ starts, int reverse) {
  GDR_POISON_ALL();
  constexpr int NJ = D / 64, NI = BV / 16, LDP = D + 4, NT = 256;
  __shared__ __align__(16) float Ps[D * LDP];   // linear part, rows k, columns j
  __shared__ __align__(16) float Wl[BV * LDP];  // this tile's rows of the running memory
  int sq, h, vt;
  if (!scan_block(geo, D / BV, sq, h, vt)) return;
  const int i0 = vt * BV, w = wave_id();
  const SeqPos sp = seq_pos(geo, sq);
  const long mem = (long)sq * geo.H + h;
  const int nseg = seg_count(sg, sp.nchunks);

  f32x4 S[NJ][NI];  // W^T tiles: rows j (key), columns i (value), as in the scans
#pragma unroll
  for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int j0 = acc_row(16 * (w + 4 * qq), 0), i = i0 + acc_col(16 * it);
      if (init) {
        const float4 x = *reinterpret_cast<const float4*>(init + (mem * D + i) * D + j0);
        S[qq][it] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        S[qq][it] = zero4();
      }
    }
  for (int kk = 0; kk < nseg; ++kk) {
    const int s = reverse ? nseg - 1 - kk : kk;
    float* st = starts + (mem * sg.max_seg + s) * D * D;
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int j0 = acc_row(16 * (w + 4 * qq), 0), i = i0 + acc_col(16 * it);
        const f32x4 x = S[qq][it];
        *reinterpret_cast<float4*>(st + (long)i * D + j0) = make_float4(x[0], x[1], x[2], x[3]);
      }
    if (kk == nseg - 1) break;
    const float* Hm = sg.maps + (mem * sg.max_seg + s) * 2 * D * D;
    const float* Pm = Hm + D * D;
    __syncthreads();
    for (int idx = threadIdx.x; idx < D * D / 4; idx += NT) {
      const int r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      *reinterpret_cast<float4*>(Ps + r * LDP + c) = *reinterpret_cast<const float4*>(Pm + (long)r * D + c);
    }
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) store4_t(Wl, LDP, 16 * (w + 4 * qq), 16 * it, S[qq][it]);
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        // (W P + H)^T tile: rows j, columns i; H rows i, four consecutive j
        const int j0 = acc_row(16 * (w + 4 * qq), 0), i = i0 + acc_col(16 * it);
        const float4 hv = *reinterpret_cast<const float4*>(Hm + (long)i * D + j0);
        f32x4 acc = f32x4{hv.x, hv.y, hv.z, hv.w};
        acc = mma_k<float, D>(acc, colk(Ps, LDP), 16 * (w + 4 * qq), rowk(Wl, LDP), 16 * it);
        S[qq][it] = acc;
      }
  }
}

template <int D, int BV>
static hipError_t seg_impl(const Plan& p, const ScanSeg& sg, const float* init, bool reverse, hipStream_t st) {
  TraceScope ts_(reverse ? "bwd_seg_combine" : "fwd_seg_combine", st);
  hipLaunchKernelGGL((k_seg_combine<D, BV>), dim3(scan_grid(p.geo, D / BV)), dim3(256), 0, st, p.geo, sg, init,
                     p.seg_starts, reverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const Plan& p, const ScanSeg& sg, const float* init, bool reverse, hipStream_t st) {
  if (p.D == 128) return p.bv == 16 ? seg_impl<128, 16>(p, sg, init, reverse, st) : seg_impl<128, 32>(p, sg, init, reverse, st);
  if (p.D == 64) return p.bv == 16 ? seg_impl<64, 16>(p, sg, init, reverse, st) : seg_impl<64, 32>(p, sg, init, reverse, st);
  return hipErrorInvalidValue;
}

}  // namespace gdr
