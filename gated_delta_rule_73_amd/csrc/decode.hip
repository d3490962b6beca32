// Recurrent (token-by-token) form of the delta-rule memory for decoding: the memory of every
// (sequence, head) is read once, takes that sequence's new tokens in order, and is written
// back once.  Per token, with D_t the decay and v_bar = (W D_t) k the memory's prediction:
//   Delta family:     W <- W D_t + beta (v - v_bar) k^T
//   Gated DeltaNet-2: W <- W D_t - v_bar (beta e*k)^T + (beta w*v) k^T
//   erase-free (GLA): W <- W D_t + beta v k^T   (D_t per key channel, nothing predicted)
//   o_t = scale * W q_t   (the memory after the token's write)
// Every value row i of W evolves on its own: v_bar_i needs only row i and k, and the write
// touches row i only through v_i, w_i and v_bar_i.  So the rows are spread over the lanes with
// no exchange beyond a sum along each row, and the kernel streams the float32 memory at HBM
// speed: each lane holds four consecutive key columns of a row (one 16-byte load and store),
// a row is a group of d_k/4 adjacent lanes, and a workgroup covers consecutive rows.  Four rows
// per lane keep four 16-byte loads in flight per lane (measured faster than one or two rows,
// and than non-temporal loads and stores of the memory).
#include "chunk.hpp"
#include "launch.hpp"

namespace gdr {

namespace {

// Sum over the LPR adjacent lanes that hold one row (LPR a power of two dividing 64).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p) {
  if constexpr (std::is_same<E, float>::value) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    return f32x4{x.x, x.y, x.z, x.w};
  } else {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  }
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

}  // namespace

// Grid: one workgroup per (memory, block of RPB value rows), memory = sequence * H + head.
// LOG: the gates are logits (beta, e, w = sigmoid(x), alpha = exp(-softplus(x))).
template <typename E, int D, int VAR, bool LOG>
__global__ __launch_bounds__(256) void k_decode(Geo geo, const E* __restrict__ q, const E* __restrict__ k,
                                                const E* __restrict__ v, const E* __restrict__ beta,
                                                const E* __restrict__ alpha, const E* __restrict__ erase,
                                                const E* __restrict__ write, float* __restrict__ state,
                                                E* __restrict__ o) {
  GDR_POISON_ALL();
  constexpr int LPR = D / 4;          // lanes per row
  constexpr int GROUPS = 256 / LPR;   // rows in flight per workgroup pass
  constexpr int RPT = 4;              // rows per lane
  constexpr int RPB = GROUPS * RPT;   // rows per workgroup
  constexpr int NRB = D / RPB;        // workgroups per memory
  static_assert(D % RPB == 0, "row blocks tile the memory");
  const int mem = blockIdx.x / NRB, rb = blockIdx.x % NRB;
  const int sq = mem / geo.H, h = mem % geo.H;
  const int j0 = 4 * (threadIdx.x % LPR), grp = threadIdx.x / LPR;
  int b = sq, bos = 0, len = geo.T;
  if (geo.varlen) {
    b = 0;
    bos = geo.cu[sq];
    len = geo.cu[sq + 1] - bos;
  }
  float* Wm = state + (long)mem * D * D;
  int row[RPT];
  f32x4 W[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    row[r] = rb * RPB + r * GROUPS + grp;
    const float4 x = *reinterpret_cast<const float4*>(Wm + (long)row[r] * D + j0);
    W[r] = f32x4{x.x, x.y, x.z, x.w};
  }
  for (int t = 0; t < len; ++t) {
    const long tk = tok_index(geo, b, h, bos + t);
    const f32x4 kt = load4(k + tk * D + j0);
    const f32x4 qt = load4(q + tk * D + j0);
    float bt = beta ? (float)beta[tk] : 1.f;
    if constexpr (LOG) bt = gate_sigmoid(bt);
    f32x4 dec = {1.f, 1.f, 1.f, 1.f};
    if constexpr (VAR == VAR_KDA || VAR == VAR_GLA) {
      dec = load4(alpha + tk * D + j0);
      if constexpr (LOG) {
#pragma unroll
        for (int x = 0; x < 4; ++x) dec[x] = expf(gate_neg_softplus(dec[x]));
      }
    } else if constexpr (VAR != VAR_DELTANET) {
      const float a = LOG ? expf(gate_neg_softplus((float)alpha[tk])) : (float)alpha[tk];
      dec = f32x4{a, a, a, a};
    }
    f32x4 ek = kt;  // direction along which the prediction is erased: beta (e*k), or beta k
    if constexpr (VAR == VAR_GDN2) {
      f32x4 e = load4(erase + tk * D + j0);
      if constexpr (LOG) {
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = gate_sigmoid(e[x]);
      }
      ek = kt * e;
    }
    ek *= bt;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4 Wd = W[r] * dec;
      float stored = bt * (float)v[tk * D + row[r]];  // beta v_i, or beta w_i v_i
      if constexpr (VAR == VAR_GDN2) {
        const float wr = (float)write[tk * D + row[r]];
        stored *= LOG ? gate_sigmoid(wr) : wr;
      }
      if constexpr (VAR == VAR_GLA) {
        W[r] = Wd + stored * kt;
      } else {
        const float vbar = row_sum<LPR>(dot4(Wd, kt));
        W[r] = Wd - vbar * ek + stored * kt;
      }
      const float ov = row_sum<LPR>(dot4(W[r], qt));
      if (j0 == 0) o[tk * D + row[r]] = (E)(geo.scale * ov);
    }
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    *reinterpret_cast<float4*>(Wm + (long)row[r] * D + j0) = float4{W[r][0], W[r][1], W[r][2], W[r][3]};
}

namespace {

template <typename E, int D>
hipError_t launch_decode_t(const Geo& g, int variant, int gates, const gdr_inputs& in, float* state, void* o,
                           hipStream_t st) {
  constexpr int RPB = 4 * 256 / (D / 4);
  const long blocks = (long)g.nseq * g.H * (D / RPB);
  if (blocks == 0) return hipSuccess;
  auto go = [&](auto kern) {
    TraceScope ts("decode", st);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, g, (const E*)in.q, (const E*)in.k,
                       (const E*)in.v, (const E*)in.beta, (const E*)in.alpha, (const E*)in.erase,
                       (const E*)in.write, state, (E*)o);
    return hipGetLastError();
  };
  if (gates) {  // gates given as logits
    switch (variant) {
      case GDR_DELTANET: return go(k_decode<E, D, VAR_DELTANET, true>);
      case GDR_GATED: return go(k_decode<E, D, VAR_GATED, true>);
      case GDR_KDA: return go(k_decode<E, D, VAR_KDA, true>);
      case GDR_GLA: return go(k_decode<E, D, VAR_GLA, true>);
      default: return go(k_decode<E, D, VAR_GDN2, true>);
    }
  }
  switch (variant) {
    case GDR_DELTANET: return go(k_decode<E, D, VAR_DELTANET, false>);
    case GDR_GATED: return go(k_decode<E, D, VAR_GATED, false>);
    case GDR_KDA: return go(k_decode<E, D, VAR_KDA, false>);
    case GDR_GLA: return go(k_decode<E, D, VAR_GLA, false>);
    default: return go(k_decode<E, D, VAR_GDN2, false>);
  }
}

}  // namespace

hipError_t run_decode(const Geo& g, int variant, int gates, int dtype, int D, const gdr_inputs& in, float* state,
                      void* o, hipStream_t st) {
  if (dtype == GDR_BF16) {
    return D == 64 ? launch_decode_t<bf16, 64>(g, variant, gates, in, state, o, st)
                   : launch_decode_t<bf16, 128>(g, variant, gates, in, state, o, st);
  }
  return D == 64 ? launch_decode_t<float, 64>(g, variant, gates, in, state, o, st)
                 : launch_decode_t<float, 128>(g, variant, gates, in, state, o, st);
}

}  // namespace gdr
