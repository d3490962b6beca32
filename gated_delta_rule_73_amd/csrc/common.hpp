// Device building blocks shared by the gfx950 kernels of the chunked delta-rule operator.
//
// Matrix products use the CDNA3/4 matrix cores through 16x16 output tiles:
//   bfloat16 operands: v_mfma_f32_16x16x32_bf16 (k = 32 per instruction, 8 values per lane)
//   float32 operands : v_mfma_f32_16x16x4_f32   (k = 4 per instruction, 1 value per lane)
// Lane l of a 64-wide wave holds, for an output tile C[m0..m0+15][n0..n0+15]:
//   A fragment: row m0 + (l & 15), k = k0 + KPL * (l >> 4) + e, e < KPL
//   B fragment: column n0 + (l & 15), same k
//   accumulator element r: row m0 + 4 * (l >> 4) + r, column n0 + (l & 15).
// Operands are read from LDS through View<S, KC>: element (m, k) lives at p[m*ld + k] when
// KC (k contiguous: one vector load per fragment) and at p[k*ld + m] otherwise (a gather).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length (tokens)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// LDS poisoning, debug builds only (GDR_LDS_POISON; the release library compiles both to
// nothing).  LDS keeps whatever the previous workgroup on the CU left there, so a read of an
// element this workgroup never wrote (or of a region whose contents are dead) is a latent bug
// even where the release build happens to get a finite value.  Poisoned bytes are 0xFF, a NaN in
// bfloat16 and in float32, so such a read shows up as NaN in the results.  Both calls are made
// by every thread of the block and are bracketed by block barriers.
//   GDR_POISON_ALL():       the kernel's whole static LDS allocation (at entry; the scans also
//                           between chunk steps, where nothing in LDS is carried over).
//   GDR_POISON(p, bytes):   one LDS region (bytes a multiple of 4) whose contents are dead.
#ifdef GDR_LDS_POISON
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ void lds_poison_all() {
  __syncthreads();
  const unsigned n = __builtin_amdgcn_groupstaticsize() / 4;  // static LDS starts at address 0
  for (unsigned i = threadIdx.x; i < n; i += blockDim.x) *(lds_u32*)(size_t)(4u * i) = 0xFFFFFFFFu;
  __syncthreads();
}
__device__ __forceinline__ void lds_poison(void* p, int bytes) {
  __syncthreads();
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
  __syncthreads();
}
#define GDR_POISON_ALL() lds_poison_all()
#define GDR_POISON(p, bytes) lds_poison((p), (bytes))
#else
#define GDR_POISON_ALL() ((void)0)
#define GDR_POISON(p, bytes) ((void)0)
#endif

// f(std::integral_constant<int, I>{}) for I = A .. B-1 in order: the body sees its index as a
// compile-time constant, so register arrays it indexes stay in registers.
template <int A, int B, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(std::integral_constant<int, A>{});
    static_for<A + 1, B>(f);
  }
}
__device__ __forceinline__ int lrow() { return threadIdx.x & 15; }
__device__ __forceinline__ int lgrp() { return (threadIdx.x >> 4) & 3; }

template <typename E> struct MMA;
template <> struct MMA<bf16> {
  static constexpr int KS = 32, KPL = 8;
  using frag = bf16x8;
  __device__ static __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MMA<float> {
  static constexpr int KS = 4, KPL = 1;
  using frag = float;
  __device__ static __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Row padding (elements) that keeps 16-byte alignment and spreads LDS banks.
template <typename S> constexpr int pad16() { return 16 / (int)sizeof(S); }

template <typename S, bool KC> struct View {
  const S* p;
  int ld;
  __device__ __forceinline__ View(const S* p_, int ld_) : p(p_), ld(ld_) {}
  __device__ __forceinline__ float at(int m, int k) const {
    return (float)(KC ? p[m * ld + k] : p[k * ld + m]);
  }
};

template <typename S> __device__ __forceinline__ View<S, true> rowk(const S* p, int ld) { return View<S, true>(p, ld); }
template <typename S> __device__ __forceinline__ View<S, false> colk(const S* p, int ld) { return View<S, false>(p, ld); }

// Row-major float data with column k scaled by sc[k]: element (m, k) = p[m*ld + k] * sc[k].
struct RowKScaled {
  const float* p;
  int ld;
  const float* sc;
  __device__ __forceinline__ float at(int m, int k) const { return p[m * ld + k] * sc[k]; }
};

// The calling lane's fragment of rows/columns idx0..idx0+15 and k-slice k0..k0+KS-1.
template <typename E, typename S, bool KC>
__device__ __forceinline__ typename MMA<E>::frag frag(const View<S, KC>& v, int idx0, int k0) {
  constexpr int KPL = MMA<E>::KPL;
  const int m = idx0 + lrow();
  const int k = k0 + KPL * lgrp();
  if constexpr (KPL == 1) {
    return (E)v.at(m, k);
  } else if constexpr (KC && std::is_same<S, E>::value) {
    return *reinterpret_cast<const bf16x8*>(v.p + m * v.ld + k);
  } else if constexpr (KC && std::is_same<S, float>::value) {
    const float4 lo = *reinterpret_cast<const float4*>(v.p + m * v.ld + k);
    const float4 hi = *reinterpret_cast<const float4*>(v.p + m * v.ld + k + 4);
    bf16x8 r;
    r[0] = (bf16)lo.x; r[1] = (bf16)lo.y; r[2] = (bf16)lo.z; r[3] = (bf16)lo.w;
    r[4] = (bf16)hi.x; r[5] = (bf16)hi.y; r[6] = (bf16)hi.z; r[7] = (bf16)hi.w;
    return r;
  } else if constexpr (!KC && std::is_same<S, E>::value) {
    // k-major bf16 data in LDS: two transposing 64-bit reads.  Within each group of 16
    // lanes, lane s addresses row k0 + 8*lgrp + s/4 (+4 for the second read), columns
    // idx0 + 4*(s%4) .. +3, and lane i receives that group's column idx0 + i for the four
    // rows -- exactly this lane's k-slice of the fragment.
    const int s = lrow();
    const S* base = v.p + (k0 + 8 * lgrp() + (s >> 2)) * v.ld + idx0 + 4 * (s & 3);
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * v.ld));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  } else {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)v.at(m, k + e);
    return r;
  }
}

template <typename E>
__device__ __forceinline__ typename MMA<E>::frag frag(const RowKScaled& v, int idx0, int k0) {
  constexpr int KPL = MMA<E>::KPL;
  const int m = idx0 + lrow(), k = k0 + KPL * lgrp();
  if constexpr (KPL == 1) {
    return (E)v.at(m, k);
  } else {
    const float4 lo = *reinterpret_cast<const float4*>(v.p + m * v.ld + k);
    const float4 hi = *reinterpret_cast<const float4*>(v.p + m * v.ld + k + 4);
    const float4 slo = *reinterpret_cast<const float4*>(v.sc + k);
    const float4 shi = *reinterpret_cast<const float4*>(v.sc + k + 4);
    bf16x8 r;
    r[0] = (bf16)(lo.x * slo.x); r[1] = (bf16)(lo.y * slo.y); r[2] = (bf16)(lo.z * slo.z); r[3] = (bf16)(lo.w * slo.w);
    r[4] = (bf16)(hi.x * shi.x); r[5] = (bf16)(hi.y * shi.y); r[6] = (bf16)(hi.z * shi.z); r[7] = (bf16)(hi.w * shi.w);
    return r;
  }
}

// acc += A[m0.., 0..K) * B[0..K), n0..] for one 16x16 tile.
template <typename E, int K, class VA, class VB>
__device__ __forceinline__ f32x4 mma_k(f32x4 acc, const VA& A, int m0, const VB& B, int n0) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += MMA<E>::KS) acc = MMA<E>::run(frag<E>(A, m0, k0), frag<E>(B, n0, k0), acc);
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A[m0.., k0..k0+16) * B[k0..k0+16, n0..] for one 16x16 tile: a product over exactly
// 16 values of k (bfloat16: v_mfma_f32_16x16x16_bf16, 4 values of k per lane at
// k0 + 4*lgrp; float32: four 16x16x4 steps).
template <typename E, class VA, class VB>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const VA& A, int m0, const VB& B, int n0, int k0) {
  if constexpr (std::is_same<E, float>::value) {
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4) acc = MMA<float>::run(frag<float>(A, m0, k0 + kk), frag<float>(B, n0, k0 + kk), acc);
    return acc;
  } else {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    auto f4 = [](const auto& v, int idx0, int kb) -> s16x4 {
      using Vw = std::decay_t<decltype(v)>;
      const int s = lrow();
      if constexpr (std::is_same<Vw, View<bf16, true>>::value) {
        return *reinterpret_cast<const s16x4*>(v.p + (idx0 + s) * v.ld + kb + 4 * lgrp());
      } else if constexpr (std::is_same<Vw, View<bf16, false>>::value) {
        // lane s of each 16-lane group addresses row kb + 4*lgrp + s/4, columns idx0 + 4*(s%4);
        // lane i receives column idx0 + i of those four rows.
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const bf16* base = v.p + (kb + 4 * lgrp() + (s >> 2)) * v.ld + idx0 + 4 * (s & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
      } else {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (bf16)v.at(idx0 + s, kb + 4 * lgrp() + e);
        return __builtin_bit_cast(s16x4, r);
      }
    };
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(f4(A, m0, k0), f4(B, n0, k0), acc, 0, 0, 0);
  }
}

// Row / column of accumulator element r of a tile at (m0, n0).
__device__ __forceinline__ int acc_row(int m0, int r) { return m0 + 4 * lgrp() + r; }
__device__ __forceinline__ int acc_col(int n0) { return n0 + lrow(); }

// Store 4 accumulator values that are consecutive along the tile's rows as 4 consecutive
// elements (row-of-output becomes the contiguous index): dst[col*ld + row0 .. row0+3].
template <typename S>
__device__ __forceinline__ void store4_t(S* dst, int ld, int m0, int n0, f32x4 v) {
  S* p = dst + acc_col(n0) * ld + m0 + 4 * lgrp();
  if constexpr (std::is_same<S, float>::value) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x4 b;
    b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4*>(p) = b;
  }
}
// Four consecutive elements dst[0..3] = v (one 8-byte bfloat16 or 16-byte float store).
template <typename S>
__device__ __forceinline__ void put4(S* dst, f32x4 v) {
  if constexpr (std::is_same<S, float>::value) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x4 b;
    b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4*>(dst) = b;
  }
}
// Four consecutive elements src[0..3] as float.
template <typename S>
__device__ __forceinline__ f32x4 get4(const S* src) {
  if constexpr (std::is_same<S, float>::value) {
    const float4 x = *reinterpret_cast<const float4*>(src);
    return f32x4{x.x, x.y, x.z, x.w};
  } else {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(src);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  }
}
// Store in the tile's own orientation: dst[row*ld + col].
template <typename S>
__device__ __forceinline__ void store4_n(S* dst, int ld, int m0, int n0, f32x4 v) {
  const int c = acc_col(n0);
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[acc_row(m0, r) * ld + c] = (S)v[r];
}

// ---------------------------------------------------------------------------------------
// Tile staging between global memory and LDS (16-byte vectors, whole block cooperates).
// ---------------------------------------------------------------------------------------
template <int B> struct VecT;
template <> struct VecT<16> { typedef uint4 type; };
template <> struct VecT<8> { typedef uint2 type; };
template <> struct VecT<4> { typedef uint32_t type; };
template <int B> __device__ __forceinline__ typename VecT<B>::type vzero();
template <> __device__ __forceinline__ uint4 vzero<16>() { return make_uint4(0u, 0u, 0u, 0u); }
template <> __device__ __forceinline__ uint2 vzero<8>() { return make_uint2(0u, 0u); }
template <> __device__ __forceinline__ uint32_t vzero<4>() { return 0u; }

// Raw buffer resource over [base, base + bytes): a load at an offset at or past `bytes` returns
// zero in hardware, so a ragged tile needs neither a clamp nor a select on the loaded data.
// Every caller passes the same base and size in all lanes of a wave (a workgroup's tile or gate
// row); they are read from the first lane so that the resource sits in scalar registers even
// where the compiler cannot prove it uniform, which would otherwise wrap every load in a loop
// over the distinct resources of the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, long bytes) {
  const long lim = bytes < 0x7fffffffL ? bytes : 0x7fffffffL;
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void* ub = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane((int)lim), 0x00020000);
}
template <int B> __device__ __forceinline__ typename VecT<B>::type buf_load(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ uint4 buf_load<16>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <> __device__ __forceinline__ uint2 buf_load<8>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <> __device__ __forceinline__ uint32_t buf_load<4>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// One gate element per lane, as loaded: no arithmetic on it (so nothing waits for the load until
// the value is used) and no branch around it.  A NULL gate, or a lane t >= n, reads 0.
template <typename E>
__device__ __forceinline__ uint32_t load_gate_raw(const E* g, int n, int t) {
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(g, g ? (long)n * (long)sizeof(E) : 0);
  if constexpr (sizeof(E) == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, t * 2, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, t * 4, 0, 0);
}
template <typename E>
__device__ __forceinline__ float gate_from_raw(uint32_t x) {
  if constexpr (sizeof(E) == 2) return __builtin_bit_cast(float, x << 16);  // bfloat16: the top half
  else return __builtin_bit_cast(float, x);
}

// Vector width (bytes) that spreads a tile of `bytes` over NT threads, 4..16.
constexpr int tile_vec_bytes(int bytes, int nt) {
  return bytes / nt >= 16 ? 16 : bytes / nt >= 8 ? 8 : 4;
}

// Register stage of a ROWS x COLS tile: each thread holds its share of vectors, so every
// global load of the tile is in flight before any of them is waited for.
template <typename S, int ROWS, int COLS, int NT>
struct RegTile {
  static constexpr int VB = tile_vec_bytes(ROWS * COLS * (int)sizeof(S), NT);
  static constexpr int VE = VB / (int)sizeof(S);
  static constexpr int VPR = COLS / VE;
  static constexpr int TOTAL = ROWS * VPR;
  static constexpr int IT = (TOTAL + NT - 1) / NT;
  typedef typename VecT<VB>::type V;
  static_assert(COLS % VE == 0, "row length must be a multiple of the vector width");
  V v[IT];
  // v <- G[r*gs + c] for r < nrows (zero below).  Buffer loads with the resource ending at
  // row nrows: every load is issued unconditionally and rows past the end read as zero, so
  // there is no branch around a load and no select waiting on its data.
  __device__ __forceinline__ void load(const S* g, long gs, int nrows) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(g, (long)nrows * gs * (long)sizeof(S));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = threadIdx.x + it * NT;
      const int r = idx / VPR, c = (idx % VPR) * VE;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        v[it] = buf_load<VB>(rs, (int)(((long)r * gs + c) * (long)sizeof(S)));
      } else {
        v[it] = vzero<VB>();
      }
    }
  }
  // LDS[r*ld + c] <- v
  __device__ __forceinline__ void store(S* lds, int ld) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = threadIdx.x + it * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        *reinterpret_cast<V*>(lds + r * ld + c) = v[it];
      }
    }
  }
  // G[r*gs + c] <- v, every row (a whole tile, e.g. a per-chunk copy in the workspace)
  __device__ __forceinline__ void store_global(S* g, long gs) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = threadIdx.x + it * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        *reinterpret_cast<V*>(g + (long)r * gs + c) = v[it];
      }
    }
  }
  // LDS[c*ld + r] <- v (transposed), element by element
  __device__ __forceinline__ void store_t(S* lds, int ld) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = threadIdx.x + it * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        const S* e = reinterpret_cast<const S*>(&v[it]);
#pragma unroll
        for (int i = 0; i < VE; ++i) lds[(c + i) * ld + r] = e[i];
      }
    }
  }
  __device__ __forceinline__ S elem(int it, int i) const { return reinterpret_cast<const S*>(&v[it])[i]; }
  __device__ __forceinline__ int row(int it) const { return (threadIdx.x + it * NT) / VPR; }
  __device__ __forceinline__ int col(int it) const { return ((threadIdx.x + it * NT) % VPR) * VE; }
};

// q/k L2-normalisation of a tile as it is loaded: every row of a register tile scaled to unit
// length, x / ||x||_2 over its COLS elements in float32 (a zero row, e.g. past a sequence's end,
// stays zero).  A row lives in VPR adjacent lanes, so its sum of squares is reduced inside that
// lane group.  inv, if not NULL, receives 1 / ||x|| per row (ROWS floats).
// Sum over aligned groups of N adjacent lanes (N = 8 or 16) with DPP lane exchanges (plain
// vector adds, no trip through the LDS crossbar): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  Each exchange pairs lanes symmetrically, so every lane of a
// group adds the same two operands (in either order) at every step and all of them end with
// bitwise the same total.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum_dpp(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += dpp_read<0xB1>(x);
  x += dpp_read<0x4E>(x);
  x += dpp_read<0x141>(x);
  if constexpr (N == 16) x += dpp_read<0x140>(x);
  return x;
}

// x_l + x_{l^16} + x_{l^32} + x_{l^48} in every lane: the sum over the four 16-lane rows of a wave.
__device__ __forceinline__ float sum_rows4(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void normalize_rows(RegTile<S, ROWS, COLS, NT>& t, float* inv) {
  using RT = RegTile<S, ROWS, COLS, NT>;
  static_assert(RT::VB == 16 && RT::TOTAL % NT == 0 && 64 % RT::VPR == 0, "whole rows per lane group");
#pragma unroll
  for (int it = 0; it < RT::IT; ++it) {
    S* e = reinterpret_cast<S*>(&t.v[it]);
    float ss = 0.f;
#pragma unroll
    for (int x = 0; x < RT::VE; ++x) {
      const float f = (float)e[x];
      ss += f * f;
    }
    ss = group_sum_dpp<RT::VPR>(ss);
    const float rn = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
    for (int x = 0; x < RT::VE; ++x) e[x] = (S)((float)e[x] * rn);
    if (inv && threadIdx.x % RT::VPR == 0) inv[t.row(it)] = rn;
  }
}

// The factors normalize_rows wrote for the rows this thread holds of a tile (inv: one float per
// row), and the tile's rows scaled by them with normalize_rows' own arithmetic: raw rows scaled
// this way are the normalised rows, bit for bit.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void load_row_factors(const RegTile<S, ROWS, COLS, NT>& t, const float* inv,
                                                 float (&rn)[RegTile<S, ROWS, COLS, NT>::IT]) {
#pragma unroll
  for (int it = 0; it < RegTile<S, ROWS, COLS, NT>::IT; ++it) rn[it] = inv[min(t.row(it), ROWS - 1)];
}
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void scale_rows(RegTile<S, ROWS, COLS, NT>& t, const float (&rn)[RegTile<S, ROWS, COLS, NT>::IT]) {
  using RT = RegTile<S, ROWS, COLS, NT>;
#pragma unroll
  for (int it = 0; it < RT::IT; ++it) {
    S* e = reinterpret_cast<S*>(&t.v[it]);
#pragma unroll
    for (int x = 0; x < RT::VE; ++x) e[x] = (S)((float)e[x] * rn[it]);
  }
}

// LDS[r*ld + c] = G[r*gs + c] for r < nrows, 0 for nrows <= r < ROWS; c < COLS.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void g2s_rows(S* lds, int ld, const S* g, long gs, int nrows) {
  RegTile<S, ROWS, COLS, NT> t;
  t.load(g, gs, nrows);
  t.store(lds, ld);
}
// The same with every row scaled by inv[row] as normalize_rows scaled it (inv NULL: a plain copy);
// the factors are loaded before the tile, so scaling waits for nothing loaded after them.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void g2s_rows_scaled(S* lds, int ld, const S* g, long gs, int nrows, const float* inv) {
  RegTile<S, ROWS, COLS, NT> t;
  float rn[RegTile<S, ROWS, COLS, NT>::IT];
  if (inv) load_row_factors(t, inv, rn);
  t.load(g, gs, nrows);
  if (inv) scale_rows(t, rn);
  t.store(lds, ld);
}
// Transposed staging: LDS[c*ld + r] = mul * G[r*gs + c] (zero for r >= nrows), r < ROWS, c < COLS.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void g2s_rows_t(S* lds, int ld, const S* g, long gs, int nrows, float mul = 1.f) {
  constexpr int VE = 16 / (int)sizeof(S);
  constexpr int VPR = COLS / VE;
  constexpr int TOTAL = ROWS * VPR;
  constexpr int IT = (TOTAL + NT - 1) / NT;
  uint4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = threadIdx.x + it * NT;
    const int r = idx % ROWS, c = (idx / ROWS) * VE;
    v[it] = make_uint4(0u, 0u, 0u, 0u);
    if ((TOTAL % NT == 0 || idx < TOTAL) && r < nrows) v[it] = *reinterpret_cast<const uint4*>(g + (long)r * gs + c);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = threadIdx.x + it * NT;
    if (TOTAL % NT == 0 || idx < TOTAL) {
      const int r = idx % ROWS, c = (idx / ROWS) * VE;
      const S* e = reinterpret_cast<const S*>(&v[it]);
#pragma unroll
      for (int i = 0; i < VE; ++i) lds[(c + i) * ld + r] = (S)((float)e[i] * mul);
    }
  }
}
// G[r*gs + c] = LDS[r*ld + c] for r < nrows, c < COLS.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void s2g_rows(S* g, long gs, const S* lds, int ld, int nrows) {
  constexpr int VE = 16 / (int)sizeof(S);
  constexpr int VPR = COLS / VE;
  constexpr int TOTAL = ROWS * VPR;
  constexpr int IT = (TOTAL + NT - 1) / NT;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = threadIdx.x + it * NT;
    const int r = idx / VPR, c = (idx % VPR) * VE;
    if ((TOTAL % NT == 0 || idx < TOTAL) && r < nrows)
      *reinterpret_cast<uint4*>(g + (long)r * gs + c) = *reinterpret_cast<const uint4*>(lds + r * ld + c);
  }
}
// The same for a tile whose every row is written: no predicate on the stores, so the count
// of outstanding memory operations stays the same on every path.
template <typename S, int ROWS, int COLS, int NT>
__device__ __forceinline__ void s2g_full(S* g, long gs, const S* lds, int ld) {
  constexpr int VB = tile_vec_bytes(ROWS * COLS * (int)sizeof(S), NT);
  constexpr int VE = VB / (int)sizeof(S);
  constexpr int VPR = COLS / VE;
  constexpr int TOTAL = ROWS * VPR;
  typedef typename VecT<VB>::type V;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the block");
#pragma unroll
  for (int it = 0; it < TOTAL / NT; ++it) {
    const int idx = threadIdx.x + it * NT;
    const int r = idx / VPR, c = (idx % VPR) * VE;
    *reinterpret_cast<V*>(g + (long)r * gs + c) = *reinterpret_cast<const V*>(lds + r * ld + c);
  }
}

// ---------------------------------------------------------------------------------------
// Problem geometry
// ---------------------------------------------------------------------------------------
// Gates given as logits x (the problem's gates == 1): beta = sigmoid(x), alpha = exp(-softplus(x)),
// so log alpha = -softplus(x) comes without rounding alpha first.  The hardware exp2/log2 paths
// (absolute error about 1e-7 here, far below the bfloat16 step of the results) keep the
// per-channel decay of Kimi Delta Attention, 64 x d_k values per chunk, as cheap as its log.
__device__ __forceinline__ float gate_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float gate_neg_softplus(float x) {
  return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x))));
}

struct Geo {
  int B, H, T;        // batch, heads, tokens
  int nseq;           // independent sequences (B, or packed count)
  int varlen;         // 1: packed sequences, B == 1
  const int* cu;      // device offsets (varlen)
  int total_chunks;   // sum over sequences of ceil(len / 64)
  float scale;
};

// Gated DeltaNet-2's gates: the value, or (LOG) sigmoid of the logit.
template <bool LOG>
__device__ __forceinline__ float g2_gate(float x) {
  if constexpr (LOG) return gate_sigmoid(x);
  else return x;
}

struct ChunkPos {
  int b, seq, t0, n;  // batch row, sequence, first token (within [0,T)), valid tokens
};
struct SeqPos {
  int b, bos, len, gc0, nchunks;
};

// Inclusive prefix sum / total of an int over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// Packed sequences are found with the whole wave: each lane reads one sequence's offsets, a
// prefix sum over the lanes gives the sequences' first chunks, and a ballot picks the one that
// holds the chunk -- 64 sequences per round of coalesced loads, so hundreds of packed
// documents cost a few rounds instead of a serial walk over cu_seqlens.  Every lane of the
// wave must call these together (they are called at the top of each kernel, or after an exit
// taken by the whole block).
__device__ __forceinline__ ChunkPos chunk_pos(const Geo& g, int gc) {
  ChunkPos p;
  if (!g.varlen) {
    const int nt = (g.T + CH - 1) / CH;
    p.b = gc / nt;
    p.seq = p.b;
    p.t0 = (gc % nt) * CH;
    p.n = min(CH, g.T - p.t0);
    return p;
  }
  p.b = 0; p.seq = 0; p.t0 = 0; p.n = 0;
  const int l = threadIdx.x & 63;
  int off = 0;  // chunks of the sequences before this round
  for (int base = 0; base < g.nseq; base += 64) {
    const int s = base + l;
    int a = 0, e = 0, nc = 0;
    if (s < g.nseq) {
      a = g.cu[s];
      e = g.cu[s + 1];
      nc = (e - a + CH - 1) / CH;
    }
    const int incl = wave_incl_scan_i(nc);
    const int first = off + incl - nc;  // this lane's sequence starts at global chunk `first`
    const unsigned long long hit = __ballot(nc > 0 && gc >= first && gc < first + nc);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int a_s = __shfl(a, src, 64), e_s = __shfl(e, src, 64), f_s = __shfl(first, src, 64);
      // every lane holds the same values; readfirstlane tells the compiler so, which keeps the
      // addresses built from them in scalar registers (a buffer resource in vector registers
      // would need a loop over lanes around every load)
      p.seq = __builtin_amdgcn_readfirstlane(base + src);
      p.t0 = __builtin_amdgcn_readfirstlane(a_s + (gc - f_s) * CH);
      p.n = min(CH, __builtin_amdgcn_readfirstlane(e_s) - p.t0);
      return p;
    }
    off = __builtin_amdgcn_readfirstlane(off + __shfl(incl, 63, 64));
  }
  return p;
}

__device__ __forceinline__ SeqPos seq_pos(const Geo& g, int s) {
  SeqPos p;
  if (!g.varlen) {
    const int nt = (g.T + CH - 1) / CH;
    p.b = s; p.bos = 0; p.len = g.T; p.gc0 = s * nt; p.nchunks = nt;
    return p;
  }
  const int l = threadIdx.x & 63;
  int off = 0;  // chunks of the sequences before s, 64 sequences per round
  for (int base = 0; base < s; base += 64) {
    const int i = base + l;
    const int nc = i < s ? (g.cu[i + 1] - g.cu[i] + CH - 1) / CH : 0;
    off += wave_sum_i(nc);
  }
  p.b = 0;
  p.bos = g.cu[s];
  p.len = g.cu[s + 1] - g.cu[s];
  p.gc0 = __builtin_amdgcn_readfirstlane(off);  // the same in every lane (see chunk_pos)
  p.nchunks = (p.len + CH - 1) / CH;
  return p;
}

// Element offset of token t (absolute within [0,T)) of head h in a [B,H,T,d] tensor, / d.
__device__ __forceinline__ long tok_index(const Geo& g, int b, int h, int t) {
  return ((long)b * g.H + h) * g.T + t;
}

// Scan kernels use a 1-D grid (times the segment count in y for segmented scans).  Work item
// (sequence, head) sh and value tile vt run on block L with L % 8 == sh % 8, so the tiles of
// one memory land on one XCD (workgroups are dealt to the 8 XCDs round-robin) and share its
// L2 for the chunk operands they all read.
inline unsigned scan_grid(const Geo& g, int nv) {
  const unsigned nsh = (unsigned)g.nseq * (unsigned)g.H;
  return ((nsh + 7u) / 8u) * 8u * (unsigned)nv;
}
__device__ __forceinline__ bool scan_block(const Geo& g, int nv, int& seq, int& h, int& vt) {
  const int L = blockIdx.x;
  vt = (L >> 3) % nv;
  const int sh = ((L >> 3) / nv) * 8 + (L & 7);
  if (sh >= g.nseq * g.H) return false;
  seq = sh / g.H;
  h = sh % g.H;
  return true;
}

// Segmented scans.  The chunk-to-chunk map of a memory is affine, W_next = W P_c + H_c (and
// dW_prev = dW Q_c + G_c in the backward), so a sequence's chunks can be cut into segments of
// lseg chunks: mode 1 runs every segment from a zero memory (giving its additive part) and,
// in extra "virtual" value tiles, from the identity with the write term removed (giving its
// linear part); a combine kernel composes the segments' maps in order to find each segment's
// start memory; mode 2 reruns every segment from that start, writing the per-chunk results.
// Mode 3 (reverse scan only) runs one segment per sequence, part `part` counted from the end
// (segment nseg - 1 - part), from the end state that part - 1 left in maps (the final-state
// gradient for part 0), and leaves its own end state there for part + 1 (dh0 for segment 0):
// launched part after part, the parts chain into the whole scan, and the chunk kernels of a
// finished part can run while later parts scan.
// A sequence has max(1, ceil(chunks / lseg)) segments; mode 0 is the unsegmented scan.
struct ScanSeg {
  int mode;             // 0, 1, 2 or 3 as above
  int lseg, max_seg;    // chunks per segment; largest segment count of any sequence
  float* maps;          // mode 1 output: [memories][max_seg][2][D][D] (additive part, linear part);
                        // mode 3: [memories][max_seg][D][D] state at the start of each segment
  const float* starts;  // mode 2 input: [memories][max_seg][D][D] start memory of each segment
  int part;             // mode 3: the part run by this launch
};
__device__ __forceinline__ int seg_count(const ScanSeg& sg, int nchunks) {
  return max(1, (nchunks + sg.lseg - 1) / sg.lseg);
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane exchanges only (vector adds,
// no trip through the LDS crossbar): a Hillis-Steele scan inside each row of 16 lanes
// (row_shr 1, 2, 4, 8; a lane whose source lies before its row adds 0), then the rows' totals
// carried forward (row_bcast 15 adds row 0's total to row 1 and row 2's to row 3, row_bcast 31
// adds the total of rows 0-1 to rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_or_zero<0x111, 0xF>(x);
  x += dpp_or_zero<0x112, 0xF>(x);
  x += dpp_or_zero<0x114, 0xF>(x);
  x += dpp_or_zero<0x118, 0xF>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return x;
}
// Sum over the 64 lanes of a wave, returned to every lane: DPP row sums, the rows' totals
// carried into the last row as in wave_incl_scan, then lane 63 read out.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum_dpp<16>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Sum over the 16 lanes sharing lgrp() (i.e. over a tile's columns).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

}  // namespace gdr
