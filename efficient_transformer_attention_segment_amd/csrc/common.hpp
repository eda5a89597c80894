// Shared device helpers for the gfx950 Nystrom attention kernels.
//
// Matrix products run on v_mfma_f32_16x16x32_bf16 (CDNA4).  Lane layout of
// one 64-lane wave (l = lane, g = l / 16):
//   A operand (16 x 32): lane holds A[l % 16][8g + e], e = 0..7
//   B operand (32 x 16): lane holds B[8g + e][l % 16]
//   C / D     (16 x 16): lane holds C[4g + r][l % 16], r = 0..3
// Because the contraction index only has to agree between A and B, several
// kernels feed the C tile of one product straight into the next product as
// an operand by using the "paired" k order: element e of the 32-wide k step
// kk is k = 32kk + 4g + e for e < 4 and 32kk + 16 + 4g + (e - 4) for e >= 4,
// which is exactly what two stacked C tiles hold in one lane.
//
// float32 accuracy from bf16 matrix cores: a float x is split into
// hi = bf16(x) and lo = bf16(x - hi); a product uses hi*hi + hi*lo + lo*hi
// (relative error about 2^-16).  Operands that are exact in bf16 (bf16
// inputs) skip the split.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nys {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int HD = 64;     // head size d
constexpr int TAPS = 65;   // depthwise conv taps
constexpr int HALO = 32;   // TAPS / 2
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1.0e30f;  // finite "minus infinity" for running maxima

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// float32 matrix core, v_mfma_f32_16x16x4_f32: lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16]; C as above.  mma8_f32 runs eight of them over two
// 8-element fragments (element e of both operands in instruction e), so it
// contracts over k(g, e) for whatever k order the two fragments share; with
// the fragments of the bf16 products it forms the same 16 x 16 x 32 product
// in plain float32 arithmetic.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma8_f32(const float* a, const float* b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = mfma_f32(a[e], b[e], c);
  return c;
}

struct Frag2 {
  bf16x8 hi, lo;
};

// acc += A * B with NS = 1 (hi only) or NS = 3 (hi*hi + hi*lo + lo*hi).
template <int NS>
__device__ __forceinline__ f32x4 mma(const Frag2& a, const Frag2& b, f32x4 c) {
  c = mfma(a.hi, b.hi, c);
  if constexpr (NS == 3) {
    c = mfma(a.hi, b.lo, c);
    c = mfma(a.lo, b.hi, c);
  }
  return c;
}

__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ void split1(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

__device__ __forceinline__ Frag2 split8(const float* x) {
  Frag2 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    split1(x[e], h, l);
    f.hi[e] = h;
    f.lo[e] = l;
  }
  return f;
}

__device__ __forceinline__ float bf16u_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ u16 f32_to_bf16u(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
// Two floats -> two round-to-nearest-even bf16 in one word (low = a): one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max across the 16 lanes of a row (lanes sharing l / 16) with DPP
// lane permutes (VALU, no LDS crossbar round trip): quad_perm [1,0,3,2] and
// [2,3,0,1] combine each quad, row_half_mirror pairs the two quads of each
// half row, row_mirror the two halves.  Every step adds two values that the
// partner lane adds in the other order, so all 16 lanes end with the same
// bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QUAD_1032 = 0xb1, DPP_QUAD_2301 = 0x4e, DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;

__device__ __forceinline__ float sum16(float v) {
  v += dpp<DPP_QUAD_1032>(v);
  v += dpp<DPP_QUAD_2301>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  return v;
}
// Sum / max across the four lanes l, l^16, l^32, l^48 (the g groups), with
// the gfx950 row swaps (VALU, no LDS round trip): permlane16_swap pairs rows
// (0,1) and (2,3), permlane32_swap pairs rows (0,2) and (1,3).
__device__ __forceinline__ float sum_g(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_g(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  return max_g(v);
}

// ---- asynchronous global -> LDS copies (gfx950 global_load_lds, 16 bytes) --
// One wave-wide instruction copies 64 x 16 bytes: lane l's 16 bytes, read
// from its own global address, land at lds_base + 16 l.  Completion is
// tracked by the wave's vmcnt; other waves see the data after the issuing
// wave has waited and all waves have passed a barrier.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Nontemporal (streaming) store, for results that no later kernel of the
// call reads: the caches evict such lines first, ahead of the operands that
// other workgroups still re-read.  T: a scalar or an ext_vector_type vector.
template <typename T>
__device__ __forceinline__ void st_nt(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_wave_base, 16, 0, 0);
}
// The same copy with the nontemporal (streaming) cache policy, for data read
// for the last time.
__device__ __forceinline__ void dma16_nt(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_wave_base, 16, 0, 2);
}

// Landmark row groups of the B V blocks (k_bv.hpp) for I/O elements of esize
// bytes, M (padded) landmarks and head size d; the host sizes the key chunks
// and the partials with the same rule.
__host__ __device__ constexpr int bv_row_groups_for(int esize, int M, int d) {
  return (esize == 2 && d == HD && M == 128) ? 2 : 1;
}

// Element strides of a [B, H, n, 64] tensor view: batch, head and token; the
// 64 channels of a token are contiguous.  Dense [B, H, n, 64] is
// {H n 64, n 64, 64}; [B, n, H, 64] is {n H 64, 64, H 64}.
struct Strides {
  long long b, h, t;
  __host__ __device__ long long base(int bh, int H) const { return (long long)(bh / H) * b + (long long)(bh % H) * h; }
};

// s_waitcnt vmcnt(N) leaving expcnt / lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier without the memory fence that __syncthreads() carries
// (which would also drain every in-flight prefetch).  The asm statements
// keep the compiler from moving memory accesses across it; callers wait for
// the LDS writes / copies that other waves need before calling it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 4-element chunks addressed by lanes 4r + i / 4, r = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-major 64-channel bf16 tiles in LDS are stored with the 16-byte chunk
// index XOR-swizzled by the row (chunk c of row r at position c ^ (r & 7))
// so that column-chunk reads of 8 consecutive rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * HD + 8 * (chunk ^ (row & 7)); }

// ---- I/O element access (float32 or raw bfloat16 bits) -------------------
template <typename IO>
struct IOTraits;

template <>
struct IOTraits<float> {
  static constexpr int NS = 3;  // products need the hi/lo split
  // load 8 consecutive elements (32-byte aligned)
  __device__ static __forceinline__ void load8(const float* p, float* x) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ static __forceinline__ void store16(float* p, const float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  }
};

template <>
struct IOTraits<u16> {
  static constexpr int NS = 1;  // bf16 inputs are exact operands
  __device__ static __forceinline__ void load8(const u16* p, float* x) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void store16(u16* p, const float* x) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    reinterpret_cast<uint4*>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
};

// 8 floats -> operand fragment (hi, and lo when NS == 3)
template <int NS>
__device__ __forceinline__ Frag2 make_frag(const float* x) {
  if constexpr (NS == 3) {
    return split8(x);
  } else {
    Frag2 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.hi[e] = (__bf16)x[e];
    return f;
  }
}

// Where the module's bf16 projection writes the landmarks it forms in its
// epilogue (k_qkv.hpp), in the landmark pass's layout.
struct QkvLandmarks {
  float* qt;  // [B H][m][64] float32
  float* kt;
  __bf16* qt_hi;  // [B H][m][64] bf16 split of qt / kt
  __bf16* qt_lo;
  __bf16* kt_hi;
  __bf16* kt_lo;
  unsigned long long* slots;  // [B H][2]: cleared
  int n, H, m, L;             // tokens per sequence, heads, landmarks, segment length (divides 64)
  float scale;                // d^-1/4 / L
};

}  // namespace nys
