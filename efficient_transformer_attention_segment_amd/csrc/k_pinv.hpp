// Iterative Moore-Penrose inverse of the landmark kernel A.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.5:
// Z_0 = A^T / c, then n_iter times X = A Z and
// Z <- (1/4) Z (13 I - X (15 I - X (7 I - X))).  The init scale c is
// (max column sum) * (max row sum) of A, taken over every head of the call
// for the default ("original") option and per head for the exact-coefficient
// option.
//
// The iteration is kept literally (X is recomputed from A and Z every step),
// which is what keeps it self-correcting in finite precision.
//
// pinv_block<M> (M <= 128, bf16 I/O): one workgroup per head, everything on
//   chip, one or two waves per 16-row tile (see the function comment).  Two
//   row-major (chunk-swizzled) LDS regions of 16-bit planes suffice: each step
//   reads one and writes the other (M = 128 fits the 160 KB LDS).  Products are
//   single fp16 matrix-core products up to 8 iterations and split-bf16
//   products (hi*hi + hi*lo + lo*hi, relative error about 2^-16) beyond.
//
// pinv_block_f32<M> (M <= 128, float32 I/O): the same schedule on the
//   float32 matrix core with float32 matrices in LDS.  Once the iteration has
//   converged, Z approaches A^+ and a relative error e in its products grows
//   to about e * cond(A) in Z; float32 products keep the result at float32
//   accuracy where split-bf16 products would not.
//
// k_pinv_init / k_pinv_gemm (M > 128): the same iteration as a sequence of
//   batched launches, one product per launch, with the matrices in global
//   memory; the kernel boundaries are the step barriers.  Float32 products
//   for float32 I/O, split-bf16 for bf16 I/O.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "k_landmark.hpp"

namespace nys {

struct PinvArgs {
  const float* A;       // [BH][M][M]
  const float* colmax;  // [BH]
  const float* rowmax;  // [BH]
  float* Z;             // [BH][M][M] out
  float* cscale;        // [BH] out
  int BH, n_iter, init_option;
  int f16;              // bf16 I/O: 1 = single fp16 products, 0 = split bf16
  int fuse_gram;        // 1: each block forms its own head's A first (m <= 128)
  int npinv;            // pseudo-inverse blocks in the launch (<= 128: slots polled by one wave)
  int record;           // 1: also write A to global (fuse_gram; for the stage hook)
  unsigned spins;       // bound on the rendezvous polls (option 0 with fuse_gram)
  unsigned* status;     // bit 0 set when a rendezvous ran out of polls
  LandmarkArgs la;      // landmarks in, A / colmax / rowmax out (fuse_gram)
  // more than 128 landmarks at d = 64: the first npinv blocks of the B V
  // launch form A by row blocks instead (gram_rows_body)
  float* gAT;           // [BH][M][M] A^T
  u16* gA16;            // [BH][M][M] A as fp16
  float* colpart;       // [BH][M / 32][M] column sums per row block
  float* rowpart;       // [BH][M / 32] largest row sum per row block
};

// Past the bound on the rendezvous wait (a.spins polls; about a second by
// default) the scale becomes NaN, so the result is visibly wrong instead of
// hanging, and the block sets this bit of the status word, which the host
// reports.
constexpr unsigned STATUS_RENDEZVOUS_TIMEOUT = 1u;

__device__ __forceinline__ float pinv_scale(const PinvArgs& a, int bh) {
  if (a.init_option == 0) {
    float cm = 0.f, rm = 0.f;
    for (int i = threadIdx.x & 63; i < a.BH; i += 64) {
      cm = fmaxf(cm, a.colmax[i]);
      rm = fmaxf(rm, a.rowmax[i]);
    }
    cm = wave_max(cm);
    rm = wave_max(rm);
    return cm * rm;
  }
  return a.colmax[bh] * a.rowmax[bh];
}

// LDS use before the iteration starts (float offsets).  Qt and Kt are staged
// at the bottom; A (row stride M + 4), the column-sum scratch and the wave
// maxima overwrite the staging area once every wave holds its rows of A in
// registers (a barrier in between), and the iteration's regions overwrite A
// once every wave has read its A operands and its Z_0 elements (another
// barrier), so the prologue needs no more LDS than the larger of the staging
// area and A.  (At 128 landmarks this keeps a pseudo-inverse block within
// half of the CU's LDS, so a B V block fits beside it.)
template <int M, int NW>
struct ProLayout {
  static constexpr int QLD = HD + 4, ALD = M + 4, TM = M / 16;
  static constexpr int OFF_QT = 0, OFF_KT = M * QLD;  // float32 staging (float32 I/O)
  static constexpr int STAGE = 2 * M * QLD;           // floats: float32 Qt, Kt, or the four bf16 planes
  static constexpr int OFF_A = 0;
  static constexpr int OFF_CSUM = OFF_A + M * ALD;
  static constexpr int OFF_WRED = OFF_CSUM + TM * M;
  static constexpr int END = OFF_WRED + 2 * NW;
  static constexpr int BYTES = 4 * (END > STAGE ? END : STAGE);
};

// A = softmax(Qt Kt^T) for one head into LDS (store_a_lds copies it to
// global for the stage hook later), with the head's maximum column and row
// sums in wred[0], wred[1] (and in colmax / rowmax).  The landmarks come into LDS in one coalesced
// pass first, so the products read LDS instead of waiting on global loads:
// float32 Qt, Kt for float32 I/O (float32 products), and for bf16 I/O the
// bf16 hi / lo planes the landmark kernel already wrote (split-bf16
// products with no conversion work here).
template <int M, bool F32, int NW, class Ly, bool PAD>
__device__ void gram_lds(const LandmarkArgs& a, int bh, float* L) {
  constexpr int TM = M / 16, QLD = Ly::QLD, ALD = Ly::ALD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  float* const Qs = L + Ly::OFF_QT;
  float* const Ks = L + Ly::OFF_KT;
  __bf16* const Bs = reinterpret_cast<__bf16*>(L);  // planes qt_hi, qt_lo, kt_hi, kt_lo, M x 64 each (swz)
  float* const Al = L + Ly::OFF_A;
  float* const csum = L + Ly::OFF_CSUM;
  float* const wred = L + Ly::OFF_WRED;
  // every load of the staging pass is issued before the first LDS store
  constexpr int NT = 64 * NW;
  if constexpr (F32) {
    constexpr int TOT = M * (HD / 4), CNT = (TOT + NT - 1) / NT;
    const float4* qt = reinterpret_cast<const float4*>(a.qt + (size_t)bh * M * HD);
    const float4* kt = reinterpret_cast<const float4*>(a.kt + (size_t)bh * M * HD);
    float4 x[CNT], y[CNT];
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const int i = tid + k * NT;
      if (i < TOT) {
        x[k] = qt[i];
        y[k] = kt[i];
      }
    }
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const int i = tid + k * NT, row = i >> 4, c4 = i & 15;
      if (i < TOT) {
        *reinterpret_cast<float4*>(Qs + row * QLD + 4 * c4) = x[k];
        *reinterpret_cast<float4*>(Ks + row * QLD + 4 * c4) = y[k];
      }
    }
  } else {
    // the four planes, M rows of 128 bytes each with XOR-swizzled 16-byte
    // chunks (swz), copied global -> LDS by DMA: one wave instruction moves
    // 8 rows (lane l: row l / 8, LDS chunk l % 8)
    const __bf16* src[4] = {a.qt_hi, a.qt_lo, a.kt_hi, a.kt_lo};
    for (int c = wave; c < 4 * (M / 8); c += NW) {
      const int p = c / (M / 8), r8 = c % (M / 8);
      const int row = 8 * r8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (row & 7);
      dma16(src[p] + ((size_t)bh * M + row) * HD + 8 * chunk, Bs + (p * M + 8 * r8) * HD);
    }
    wait_vmcnt<0>();
  }
  __syncthreads();
  // one row tile per wave (TM <= NW); its rows of A stay in registers until
  // every wave is done with the staging area, which A then overwrites
  static_assert(TM <= NW, "one row tile of A per wave");
  float rmax_w = 0.f;
  f32x4 acc[TM];
  float cs[TM];
  const int rt = wave;
  if (rt < TM) {
    // operands: element e of lane (g, c16) is k = 32 ks + 8 g + e
    float ax[2][8];
    Frag2 af[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = 16 * rt + c16, col = 32 * ks + 8 * g;
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ax[ks][e] = Qs[row * QLD + col + e];
      } else {
        af[ks].hi = *reinterpret_cast<const bf16x8*>(Bs + swz(row, 4 * ks + g));
        af[ks].lo = *reinterpret_cast<const bf16x8*>(Bs + M * HD + swz(row, 4 * ks + g));
      }
    }
    // column tiles in pairs: both tiles' operand reads are issued before
    // their products, and the two accumulation chains interleave
#pragma unroll
    for (int c2 = 0; c2 < TM; c2 += 2) {
      if constexpr (F32) {
#pragma unroll
        for (int ct = c2; ct < c2 + 2; ++ct) {
          acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int row = 16 * ct + c16, col = 32 * ks + 8 * g;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = Ks[row * QLD + col + e];
            acc[ct] = mma8_f32(ax[ks], x, acc[ct]);
          }
        }
      } else {
        Frag2 bf[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int row = 16 * (c2 + u) + c16;
            bf[u][ks].hi = *reinterpret_cast<const bf16x8*>(Bs + 2 * M * HD + swz(row, 4 * ks + g));
            bf[u][ks].lo = *reinterpret_cast<const bf16x8*>(Bs + 3 * M * HD + swz(row, 4 * ks + g));
          }
        acc[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[c2 + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int u = 0; u < 2; ++u) acc[c2 + u] = mma<3>(af[ks], bf[u][ks], acc[c2 + u]);
      }
      // keep the next pair's operand reads from being hoisted above this
      // pair (all of them at once would not fit the register budget)
      asm volatile("" ::: "memory");
    }
    // row softmax: row 16rt + 4g + r, columns spread over ct and lane & 15;
    // (PAD) padding columns take no weight and padding rows are zero
    if constexpr (PAD) pad_mask_cols(acc, a.mr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = NEG_BIG;
#pragma unroll
      for (int ct = 0; ct < TM; ++ct) mx = fmaxf(mx, acc[ct][r]);
      mx = max16(mx);
      float s = 0.f;
#pragma unroll
      for (int ct = 0; ct < TM; ++ct) {
        const float p = fast_exp2((acc[ct][r] - mx) * LOG2E);
        acc[ct][r] = p;
        s += p;
      }
      s = sum16(s);
      const float inv = 16 * rt + 4 * g + r < a.mr ? 1.0f / s : 0.f;
      float rs = 0.f;
#pragma unroll
      for (int ct = 0; ct < TM; ++ct) {
        acc[ct][r] *= inv;
        rs += acc[ct][r];
      }
      rs = sum16(rs);
      rmax_w = fmaxf(rmax_w, rs);
    }
#pragma unroll
    for (int ct = 0; ct < TM; ++ct) cs[ct] = sum_g(acc[ct][0] + acc[ct][1] + acc[ct][2] + acc[ct][3]);
  }
  rmax_w = max_g(rmax_w);
  __syncthreads();  // the staging area is dead from here on
  if (rt < TM) {
#pragma unroll
    for (int ct = 0; ct < TM; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        Al[row * ALD + 16 * ct + c16] = acc[ct][r];
      }
      if (g == 0) csum[rt * M + 16 * ct + c16] = cs[ct];
    }
  }
  if (lane == 0) wred[wave] = rmax_w;
  __syncthreads();
  // column sums in a fixed order, then the block maximum
  float cmax = 0.f;
  for (int j = tid; j < M; j += 64 * NW) {
    float s = 0.f;
    for (int rt = 0; rt < TM; ++rt) s += csum[rt * M + j];
    cmax = fmaxf(cmax, s);
  }
  cmax = wave_max(cmax);
  if (lane == 0) wred[NW + wave] = cmax;
  __syncthreads();
  float rm = 0.f, cm = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    rm = fmaxf(rm, wred[i]);
    cm = fmaxf(cm, wred[NW + i]);
  }
  __syncthreads();
  if (tid == 0) {
    a.rowmax[bh] = rm;
    a.colmax[bh] = cm;
    wred[0] = cm;
    wred[1] = rm;
  }
  __syncthreads();
}

// c for one head's block; on return A is in LDS at Ly::OFF_A (row stride
// M + 4).  With fuse_gram the block forms A itself (gram_lds); otherwise it
// copies the A of the separate Gram launch.  Option 1 needs only this head.
// Option 0 needs the maxima over every head: the pseudo-inverse blocks are
// the first npinv blocks of the launch (dispatched first, all resident: the
// host fuses only while npinv is at most 128, half the CU count), and meet
// once.  Each publishes its two maxima as 64-bit words (valid bit 32 above
// the float bits) with single agent-scope atomic stores into its own slots,
// which the landmark launch cleared; wave 0 of every block then polls all
// slots (one 64-bit atomic load per slot, two slots per lane) until every
// one is valid, and takes the maxima.  A word is written whole, so a valid
// one carries its maximum; there is no other shared data and no fence.
template <int M, bool F32, int NW, class Ly, bool PAD>
__device__ float pinv_prologue(const PinvArgs& a, int bh, float* L) {
  float* const wred = L + Ly::OFF_WRED;
  if (!a.fuse_gram) {
    constexpr int NT = 64 * NW, TOT = M * M / 4, CNT = (TOT + NT - 1) / NT;
    const float4* A = reinterpret_cast<const float4*>(a.A + (size_t)bh * M * M);
    // every element of x is assigned (out-of-range slots read element 0 and
    // are not stored), so the array stays in registers
    float4 x[CNT];
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const int i = threadIdx.x + k * NT;
      x[k] = A[i < TOT ? i : 0];
    }
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const int i = threadIdx.x + k * NT, row = i / (M / 4), c4 = i % (M / 4);
      if (i < TOT) *reinterpret_cast<float4*>(L + Ly::OFF_A + row * Ly::ALD + 4 * c4) = x[k];
    }
    __syncthreads();
    return pinv_scale(a, bh);
  }
  gram_lds<M, F32, NW, Ly, PAD>(a.la, bh, L);
  const float cm = wred[0], rm = wred[1];
  if (a.init_option != 0) return cm * rm;
  __syncthreads();  // every thread has read wred
  constexpr unsigned long long VALID = 1ull << 32;
  unsigned long long* const slots = a.la.slots;
  if (threadIdx.x == 0) {
    __hip_atomic_store(slots + 2 * bh, VALID | __float_as_uint(cm), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slots + 2 * bh + 1, VALID | __float_as_uint(rm), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float c = __builtin_nanf("");
    bool met = false;
    for (unsigned it = 0; it < a.spins; ++it) {
      bool ok = true;
      float cmx = 0.f, rmx = 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int b = lane + 64 * k;
        if (b < a.npinv) {
          const unsigned long long v0 = __hip_atomic_load(slots + 2 * b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const unsigned long long v1 =
              __hip_atomic_load(slots + 2 * b + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = ok && (v0 & VALID) && (v1 & VALID);
          cmx = fmaxf(cmx, __uint_as_float((unsigned)v0));
          rmx = fmaxf(rmx, __uint_as_float((unsigned)v1));
        }
      }
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
        c = wave_max(cmx) * wave_max(rmx);
        met = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) {
      wred[0] = c;
      if (!met) __hip_atomic_fetch_or(a.status, STATUS_RENDEZVOUS_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  return wred[0];
}

// The A the block formed itself (fuse_gram), from LDS to global when the
// stage hook asks for it; called before the LDS copy of A is overwritten.
template <int M, int ALD>
__device__ __forceinline__ void store_a_lds(const PinvArgs& a, const float* Al, int bh) {
  if (!a.fuse_gram || !a.record) return;
  float* A = a.la.A + (size_t)bh * M * M;
  for (int i = threadIdx.x; i < M * M / 4; i += blockDim.x) {
    const int row = i / (M / 4), c4 = i % (M / 4);
    *reinterpret_cast<float4*>(A + (size_t)row * M + 4 * c4) =
        *reinterpret_cast<const float4*>(Al + row * ALD + 4 * c4);
  }
}

// Z = Z_0 = A^T / c (no iterations), from A in LDS, by the whole block.
template <int M, int ALD>
__device__ __forceinline__ void store_z0_lds(const float* Al, float* Zg, float invc) {
  for (int idx = threadIdx.x; idx < M * M; idx += blockDim.x) {
    const int row = idx / M, col = idx % M;
    Zg[idx] = Al[col * ALD + row] * invc;
  }
}

// Waves per workgroup for m landmarks: one per 16-row tile up to 128
// landmarks, two per tile (each forming half of the tile's outputs) for
// m <= 64, rounded up to a power of two (4 or 8).
template <int M>
constexpr int pinv_wpt() {
  return M <= 64 ? 2 : 1;
}
template <int M>
constexpr int nwaves() {
  return (M / 16) * pinv_wpt<M>() <= 4 ? 4 : 8;
}

// ---------------------------------------------------------------------------
// bf16-I/O variant.  Operands live in LDS as 16-bit planes, in one of two
// encodings:
//   split bf16 (F16 = false): planes hi and lo, products hi*hi + hi*lo +
//     lo*hi (relative error about 2^-16);
//   single fp16 (F16 = true): one plane, one v_mfma_f32_16x16x32_f16 per
//     product (11-bit operands, float32 accumulation): a third of the
//     matrix-core work and half the LDS traffic.
// The host takes fp16 for iteration counts up to 8: the iterate after t
// steps is a fixed polynomial of A A^T applied to A^T, so its sensitivity to
// operand rounding grows with t (a converged iterate magnifies errors by up
// to the condition number of A), and the split encoding beyond that.

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <bool F16>
struct POp;

template <>
struct POp<false> {
  static constexpr int NP = 2;  // planes
  typedef Frag2 Frag;
  __device__ static __forceinline__ Frag make(const float* x) { return split8(x); }
  __device__ static __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) { return nys::mma<3>(a, b, c); }
  __device__ static __forceinline__ void set(Frag& f, int p, s16x8 v) {
    if (p == 0)
      f.hi = __builtin_bit_cast(bf16x8, v);
    else
      f.lo = __builtin_bit_cast(bf16x8, v);
  }
  // 4 floats -> plane words
  __device__ static __forceinline__ void enc4(const f32x4 v, s16x4* w) {
    bf16x4 h, l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      __bf16 a, b;
      split1(v[r], a, b);
      h[r] = a;
      l[r] = b;
    }
    w[0] = __builtin_bit_cast(s16x4, h);
    w[1] = __builtin_bit_cast(s16x4, l);
  }
};

template <>
struct POp<true> {
  static constexpr int NP = 1;
  struct Frag {
    f16x8 v;
  };
  __device__ static __forceinline__ Frag make(const float* x) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (_Float16)x[e];
    return f;
  }
  __device__ static __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
  }
  __device__ static __forceinline__ void set(Frag& f, int, s16x8 v) { f.v = __builtin_bit_cast(f16x8, v); }
  __device__ static __forceinline__ void enc4(const f32x4 v, s16x4* w) {
    f16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (_Float16)v[r];
    w[0] = __builtin_bit_cast(s16x4, h);
  }
};

// Row stride (16-bit elements) of the bf16-I/O iteration's LDS matrices (see
// pswz).
template <int M>
constexpr int pinv_ld() {
  return M + 16;
}

template <int M, bool F16>
constexpr int pinv_lds_bytes() {
  constexpr int iter = 2 * POp<F16>::NP * M * pinv_ld<M>() * 2;  // two regions of NP planes
  constexpr int pro = ProLayout<M, nwaves<M>()>::BYTES;
  return iter > pro ? iter : pro;
}

__device__ __forceinline__ s16x4 lds_tr_raw(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

__device__ __forceinline__ s16x8 cat44(s16x4 a, s16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Matrices are row-major with row stride M + 16 elements (4 or 12 8-byte
// chunks past a multiple of 16) and the low two bits of each row's 8-byte
// chunk index XORed with (row >> 2) & 3.  The two access patterns of the
// iteration then hit 16 distinct 8-byte bank slots per 16 lanes: a
// transposed read (4 consecutive rows, aligned to 4, x 4 consecutive chunks,
// aligned to 4: the stride separates the rows) and a row read or store (16
// consecutive rows, one chunk: the stride separates row & 3, the XOR
// row >> 2).  Because only the low chunk bits are permuted, the tile and k
// step parts of every address stay plain additive offsets.
__device__ __forceinline__ int pswz(int row, int chunk) {
  return 4 * (chunk ^ ((row >> 2) & 3));
}

// A operand rows i*16 .. i*16+15 of Y^T (= columns of Y) for one 32-wide k
// step, read from Y (row stride LD, planes PL apart) with two transposed
// reads per plane.  PAIRED selects the paired k order (k = 4g + e,
// 16 + 4g + e - 4), otherwise the standard one (k = 8g + e).
template <int LD, int PL, bool PAIRED, bool F16>
__device__ __forceinline__ typename POp<F16>::Frag colfrag(const u16* Y, int i, int ks) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  // rows k0 = 32 ks + r0 and k1 = k0 + (PAIRED ? 16 : 4); chunk 4 i + (c16 & 3).
  // (k >> 2) & 3 does not depend on ks, so pswz is written out as a lane
  // part plus the additive 32 ks LD + 16 i (immediate offsets).
  const int r0 = (PAIRED ? 4 * g : 8 * g) + (c16 >> 2);
  const int r1 = r0 + (PAIRED ? 16 : 4);
  const int a0 = r0 * LD + 4 * ((c16 & 3) ^ ((r0 >> 2) & 3)) + 32 * ks * LD + 16 * i;
  const int a1 = r1 * LD + 4 * ((c16 & 3) ^ ((r1 >> 2) & 3)) + 32 * ks * LD + 16 * i;
  typename POp<F16>::Frag f;
#pragma unroll
  for (int p = 0; p < POp<F16>::NP; ++p)
    POp<F16>::set(f, p, cat44(lds_tr_raw(Y + p * PL + a0), lds_tr_raw(Y + p * PL + a1)));
  return f;
}

// Store this lane's 4 consecutive elements Y[row][col .. col+3] (col % 4 == 0).
template <int LD, int PL, bool F16>
__device__ __forceinline__ void rowstore4(u16* Y, int row, int col, const f32x4 v) {
  s16x4 w[POp<F16>::NP];
  POp<F16>::enc4(v, w);
  const int a = row * LD + 4 * (((col >> 2) & 3) ^ ((row >> 2) & 3)) + (col & ~15);  // = row LD + pswz(row, col / 4)
#pragma unroll
  for (int p = 0; p < POp<F16>::NP; ++p) *reinterpret_cast<s16x4*>(Y + p * PL + a) = w[p];
}

// B operand for the paired k step ks of row `row` of an LDS matrix:
// elements k = 32ks + 4g + e and 32ks + 16 + 4g + (e - 4).
template <int LD, int PL, bool F16>
__device__ __forceinline__ typename POp<F16>::Frag rowfrag(const u16* Y, int row, int ks) {
  const int g = (threadIdx.x & 63) >> 4;
  const int base = row * LD + 4 * (g ^ ((row >> 2) & 3));  // chunks 8 ks + g and 8 ks + 4 + g
  const int a0 = base + 32 * ks, a1 = base + 32 * ks + 16;
  typename POp<F16>::Frag f;
#pragma unroll
  for (int p = 0; p < POp<F16>::NP; ++p)
    POp<F16>::set(f, p, cat44(*reinterpret_cast<const s16x4*>(Y + p * PL + a0),
                              *reinterpret_cast<const s16x4*>(Y + p * PL + a1)));
  return f;
}

// One workgroup per head.  Wave w = (t, h) works on row group t: row tiles
// RT t .. RT t + RT - 1 (rows of X, T1, T2 and Z), and forms the output
// column tiles i = h, h + WPG, ... of each product for all of them, so every
// left-operand fragment it reads from LDS feeds RT products (RT = 2 for the
// fp16 encoding at m = 128, which halves the LDS traffic of the step; the
// split encoding keeps RT = 1 for registers).  Every product is formed
// transposed, Y^T[:, own rows] = (left)^T (own rows of the right factor)^T,
// so its C tile gives the lane 4 consecutive elements of one of its rows:
//   step 1  X^T  = Z^T A^T                      (Z read from LDS)
//   step 2  T1^T = 7 X^T - X^T X^T              (X from LDS)
//   step 3  T2^T = 15 X^T - T1^T X^T            (T1 from LDS)
//   step 4  Z'^T = (13 Z^T - T2^T Z^T) / 4      (T2 from LDS)
// which is Z' = Z (13I - X(15I - X(7I - X))) / 4 with X = A Z, expanded.
// The left operands come from LDS by transposed reads; the right operands
// are the wave's own rows (A from registers, X and Z re-read from the LDS
// copy after each barrier); X and Z also stay in float32 for the 7X, 15X
// and 13Z terms.  LDS holds the matrix each step reads whole, row-major,
// alternating between two regions.
template <int M, bool F16>
constexpr int pinv_rt() {
  return (M == 128 && F16) ? 2 : 1;
}

template <int M, bool F16, bool PAD>
__device__ void pinv_block(const PinvArgs& a, int bh, u16* lds) {
  typedef POp<F16> P;
  typedef typename P::Frag Frag;
  constexpr int TM = M / 16, KS = M / 32, LD = pinv_ld<M>(), PL = M * LD;
  constexpr int RT = pinv_rt<M, F16>();
  constexpr int WPG = RT == 2 ? 2 : pinv_wpt<M>();  // waves per row group
  constexpr int CT = TM / WPG;                       // output column tiles per wave
  static_assert((TM / RT) * WPG <= nwaves<M>(), "row groups exceed the block");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = w / WPG, h = w % WPG;
  const int g = lane >> 4, c16 = lane & 15;
  u16* const R0 = lds;
  u16* const R1 = lds + P::NP * PL;
  float* Zg = a.Z + (size_t)bh * M * M;

  using Ly = ProLayout<M, nwaves<M>()>;
  const float c = pinv_prologue<M, false, nwaves<M>(), Ly, PAD>(a, bh, reinterpret_cast<float*>(lds));
  const float invc = 1.0f / c;
  const float* const Al = reinterpret_cast<const float*>(lds) + Ly::OFF_A;  // A, row stride Ly::ALD
  if (threadIdx.x == 0) a.cscale[bh] = c;
  store_a_lds<M, Ly::ALD>(a, Al, bh);
  if (a.n_iter == 0) {
    store_z0_lds<M, Ly::ALD>(Al, Zg, invc);
    return;
  }
  const bool own = t < TM / RT;
  int rows[RT];  // the lane's rows of X, T1, T2, Z, one per row tile
#pragma unroll
  for (int r = 0; r < RT; ++r) rows[r] = 16 * (RT * t + r) + c16;

  Frag Af[RT][KS], Xf[RT][KS], Zf[RT][KS];
  f32x4 Xacc[RT][CT], Zacc[RT][CT], acc[RT][CT];
  // With one wave per row group (WPG == 1) the wave's C tiles hold all of its
  // own rows: tiles 2 ks and 2 ks + 1 are exactly the paired-order elements
  // of k step ks, so the own-row operands are encoded from the float32
  // accumulators (the same values the LDS copy was encoded from) instead of
  // being kept in registers or read back.
  auto own_frags = [&](const f32x4 (&src)[RT][CT], Frag (&dst)[RT][KS]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float x[8] = {src[r][2 * ks][0],     src[r][2 * ks][1],     src[r][2 * ks][2],
                            src[r][2 * ks][3],     src[r][2 * ks + 1][0], src[r][2 * ks + 1][1],
                            src[r][2 * ks + 1][2], src[r][2 * ks + 1][3]};
        dst[r][ks] = P::make(x);
      }
  };
  if (own) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // 8 consecutive floats of a row (16-byte aligned: the row stride is a
        // multiple of 4 floats)
        const float4* ap = reinterpret_cast<const float4*>(Al + rows[r] * Ly::ALD + 32 * ks + 8 * g);
        const float4 u = ap[0], v = ap[1];
        const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        Af[r][ks] = P::make(x);
      }
    // Z_0 = A^T / c: Zacc[r][j][q] = Z_0[rows[r]][16i + 4g + q], i = h + WPG j
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const int i = h + WPG * j;
#pragma unroll
        for (int q = 0; q < 4; ++q) Zacc[r][j][q] = Al[(16 * i + 4 * g + q) * Ly::ALD + rows[r]] * invc;
      }
  }
  __syncthreads();  // A is dead: R0 overwrites it
  if (own) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int j = 0; j < CT; ++j) rowstore4<LD, PL, F16>(R0, rows[r], 16 * (h + WPG * j) + 4 * g, Zacc[r][j]);
  }
  __syncthreads();

  // acc[r][j] = (left^T column tile i) x Rf[r]: PAIRED selects the k order
  // of the left operand to match Rf
  auto product = [&](const u16* Lsrc, const Frag (&Rf)[RT][KS], auto paired) {
#pragma unroll
    for (int j = 0; j < CT; ++j) {
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag lf = colfrag<LD, PL, decltype(paired)::value, F16>(Lsrc, h + WPG * j, ks);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][j] = P::mma(lf, Rf[r][ks], acc[r][j]);
      }
      // split operands at 128 landmarks: keep the next column tile's reads
      // from being hoisted above this one (they would not fit beside the
      // iteration's live fragments and accumulators, and spilled)
      if constexpr (!F16 && M > 64) asm volatile("" ::: "memory");
    }
  };
  using Std = std::integral_constant<bool, false>;
  using Pair = std::integral_constant<bool, true>;

  for (int it = 0; it < a.n_iter; ++it) {
    const bool last = (it == a.n_iter - 1);
    if (own) {  // step 1: X^T = Z^T A^T; Z's own rows kept for step 4
      if constexpr (WPG > 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) Zf[r][ks] = rowfrag<LD, PL, F16>(R0, rows[r], ks);
      }
      product(R0, Af, Std{});
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          Xacc[r][j] = acc[r][j];
          rowstore4<LD, PL, F16>(R1, rows[r], 16 * (h + WPG * j) + 4 * g, acc[r][j]);
        }
    }
    __syncthreads();
    if (own) {  // step 2: T1^T = 7 X^T - X^T X^T
      if constexpr (WPG > 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) Xf[r][ks] = rowfrag<LD, PL, F16>(R1, rows[r], ks);
      } else {
        own_frags(Xacc, Xf);
      }
      product(R1, Xf, Pair{});
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
          rowstore4<LD, PL, F16>(R0, rows[r], 16 * (h + WPG * j) + 4 * g, 7.f * Xacc[r][j] - acc[r][j]);
    }
    __syncthreads();
    if (own) {  // step 3: T2^T = 15 X^T - T1^T X^T
      if constexpr (WPG == 1) own_frags(Xacc, Xf);
      product(R0, Xf, Pair{});
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
          rowstore4<LD, PL, F16>(R1, rows[r], 16 * (h + WPG * j) + 4 * g, 15.f * Xacc[r][j] - acc[r][j]);
    }
    __syncthreads();
    if (own) {  // step 4: Z'^T = (13 Z^T - T2^T Z^T) / 4
      if constexpr (WPG == 1) own_frags(Zacc, Zf);
      product(R1, Zf, Pair{});
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          Zacc[r][j] = 0.25f * (13.f * Zacc[r][j] - acc[r][j]);
          const int col = 16 * (h + WPG * j) + 4 * g;
          if (last)
            *reinterpret_cast<float4*>(Zg + (size_t)rows[r] * M + col) =
                make_float4(Zacc[r][j][0], Zacc[r][j][1], Zacc[r][j][2], Zacc[r][j][3]);
          else
            rowstore4<LD, PL, F16>(R0, rows[r], col, Zacc[r][j]);
        }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// float32 variant.  The same waves, tiles and four steps, in the direct
// orientation: wave (t, h) forms Y[16t .. 16t+15][16i .. 16i+15] for its
// tiles i = h, h + WPT, ... as (own rows of the left factor) x (right
// factor), so the C tile gives the lane 4 consecutive rows of one column.
// Every matrix is therefore kept in LDS transposed (Y^T row-major, row
// stride M + 4): a C tile is one 16-byte store, a right-factor operand (a
// column of Y) is two 16-byte reads, and the own-row operands (rows of Z and
// X, read once per iteration) are strided single reads; the stride M + 4
// keeps both patterns free of bank conflicts.  Fragment element e of lane
// group g is k = 32ks + 4g + e (e < 4) or 32ks + 16 + 4g + (e - 4).

template <int M>
constexpr int pinv_lds_bytes_f32() {
  constexpr int iter = 2 * M * (M + 4) * 4;  // two float32 regions, row stride M + 4
  constexpr int pro = ProLayout<M, nwaves<M>()>::BYTES;
  return iter > pro ? iter : pro;
}

__device__ __forceinline__ int pk(int ks, int g, int e) { return 32 * ks + (e < 4 ? 4 * g + e : 12 + 4 * g + e); }

// Own-row operand: row `row` of Y, from Y^T stored with row stride LD.
template <int LD>
__device__ __forceinline__ void rowop_t(const float* R, int row, int ks, float* f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = R[pk(ks, g, e) * LD + row];
}

// Right-factor operand: column `col` of Y = row `col` of Y^T (contiguous).
template <int LD>
__device__ __forceinline__ void colop_t(const float* R, int col, int ks, float* f) {
  const int g = (threadIdx.x & 63) >> 4;
  const float* p = R + col * LD + 32 * ks + 4 * g;
  const float4 u = *reinterpret_cast<const float4*>(p);
  const float4 v = *reinterpret_cast<const float4*>(p + 16);
  f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
}

// C tile element (row0 + 4g + r, col) for r = 0..3 into Y^T.
template <int LD>
__device__ __forceinline__ void store_t(float* R, int col, int row4, const f32x4 v) {
  *reinterpret_cast<float4*>(R + col * LD + row4) = make_float4(v[0], v[1], v[2], v[3]);
}

template <int M, bool PAD>
__device__ void pinv_block_f32(const PinvArgs& a, int bh, float* lds) {
  constexpr int TM = M / 16, KS = M / 32, LD = M + 4;
  constexpr int WPT = pinv_wpt<M>();
  constexpr int NI = TM / WPT;  // output tiles per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = w / WPT, h = w % WPT;
  const int g = lane >> 4, c16 = lane & 15;
  float* const R0 = lds;
  float* const R1 = lds + M * LD;
  float* Zg = a.Z + (size_t)bh * M * M;

  using Ly = ProLayout<M, nwaves<M>()>;
  const float c = pinv_prologue<M, true, nwaves<M>(), Ly, PAD>(a, bh, lds);
  const float invc = 1.0f / c;
  const float* const Al = lds + Ly::OFF_A;  // A, row stride Ly::ALD
  if (threadIdx.x == 0) a.cscale[bh] = c;
  store_a_lds<M, Ly::ALD>(a, Al, bh);
  if (a.n_iter == 0) {
    store_z0_lds<M, Ly::ALD>(Al, Zg, invc);
    return;
  }
  const bool own = t < TM;
  const int row0 = 16 * t;            // the wave's rows of X, T1, T2, Z
  const int row = row0 + c16;         // the lane's row in A-operand fragments
  const int row4 = row0 + 4 * g;      // first of the lane's 4 C-tile rows

  float Af[KS][8], Xf[KS][8], Zf[KS][8];
  f32x4 Xacc[NI], Zacc[NI], acc[NI];
  if (own) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float* p = Al + row * Ly::ALD + 32 * ks + 4 * g;
      const float4 u = *reinterpret_cast<const float4*>(p);
      const float4 v = *reinterpret_cast<const float4*>(p + 16);
      Af[ks][0] = u.x; Af[ks][1] = u.y; Af[ks][2] = u.z; Af[ks][3] = u.w;
      Af[ks][4] = v.x; Af[ks][5] = v.y; Af[ks][6] = v.z; Af[ks][7] = v.w;
    }
    // Z_0 = A^T / c: Zacc[j][r] = Z_0[row4 + r][16i + c16] = A[16i + c16][row4 + r] / c,
    // and Z_0^T = A / c goes to LDS.
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = 16 * (h + WPT * j) + c16;
      const float4 z = *reinterpret_cast<const float4*>(Al + col * Ly::ALD + row4);
      Zacc[j] = f32x4{z.x * invc, z.y * invc, z.z * invc, z.w * invc};
    }
  }
  __syncthreads();  // A is dead: R0 overwrites it
  if (own) {
#pragma unroll
    for (int j = 0; j < NI; ++j) store_t<LD>(R0, 16 * (h + WPT * j) + c16, row4, Zacc[j]);
  }
  __syncthreads();

  for (int it = 0; it < a.n_iter; ++it) {
    const bool last = (it == a.n_iter - 1);
    if (own) {  // step 1: X = A Z; Z's own rows kept for step 4
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) rowop_t<LD>(R0, row, ks, Zf[ks]);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = 16 * (h + WPT * j) + c16;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float b[8];
          colop_t<LD>(R0, col, ks, b);
          acc[j] = mma8_f32(Af[ks], b, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        Xacc[j] = acc[j];
        store_t<LD>(R1, 16 * (h + WPT * j) + c16, row4, acc[j]);
      }
    }
    __syncthreads();
    if (own) {  // step 2: T1 = 7 X - X X
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) rowop_t<LD>(R1, row, ks, Xf[ks]);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = 16 * (h + WPT * j) + c16;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float b[8];
          colop_t<LD>(R1, col, ks, b);
          acc[j] = mma8_f32(Xf[ks], b, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) store_t<LD>(R0, 16 * (h + WPT * j) + c16, row4, 7.f * Xacc[j] - acc[j]);
    }
    __syncthreads();
    if (own) {  // step 3: T2 = 15 X - X T1
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = 16 * (h + WPT * j) + c16;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float b[8];
          colop_t<LD>(R0, col, ks, b);
          acc[j] = mma8_f32(Xf[ks], b, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) store_t<LD>(R1, 16 * (h + WPT * j) + c16, row4, 15.f * Xacc[j] - acc[j]);
    }
    __syncthreads();
    if (own) {  // step 4: Z' = (13 Z - Z T2) / 4
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = 16 * (h + WPT * j) + c16;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float b[8];
          colop_t<LD>(R1, col, ks, b);
          acc[j] = mma8_f32(Zf[ks], b, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        Zacc[j] = 0.25f * (13.f * Zacc[j] - acc[j]);
        const int col = 16 * (h + WPT * j) + c16;
        if (last) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Zg[(size_t)(row4 + r) * M + col] = Zacc[j][r];
        } else {
          store_t<LD>(R0, col, row4, Zacc[j]);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// M > 128: the iteration as a launch sequence over global memory.

// grid: BH blocks of 256: c, then Z = A^T / c.
// grid ((M/32)^2, BH), block 256: c, then the 32 x 32 tile (tr, tc) of
// Z = A^T / c through an LDS tile (coalesced reads and writes).
static __global__ __launch_bounds__(256) void k_pinv_init(PinvArgs a, int M) {
  __shared__ float tile[32][33];
  const int bh = blockIdx.y;
  const int nb = M / 32;
  const int tr = blockIdx.x / nb, tc = blockIdx.x % nb;
  const float c = pinv_scale(a, bh);
  const float invc = 1.0f / c;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.cscale[bh] = c;
  const float* A = a.A + (size_t)bh * M * M;
  float* Z = a.Z + (size_t)bh * M * M;
  const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
  for (int y = y0; y < 32; y += 8) tile[y][x] = A[(size_t)(32 * tc + y) * M + 32 * tr + x];  // A rows of Z's columns
  __syncthreads();
  for (int y = y0; y < 32; y += 8) Z[(size_t)(32 * tr + y) * M + 32 * tc + x] = tile[x][y] * invc;
}

// C = alpha * P * Q' with Q' = Q when beta == 0, else beta * I - Q.
// grid: ((M/32)^2, BH), block 256 (4 waves, one 16x16 tile each).  F32:
// float32 matrix-core products (float32 I/O), else split-bf16 products.  M
// is a compile-time size so the k loop unrolls and every operand load is
// issued before the first product (one round trip, not one per k step).
template <bool F32, int M>
__global__ __launch_bounds__(256) void k_pinv_gemm(const float* __restrict__ P, const float* __restrict__ Q,
                                                    float* __restrict__ C, float beta, float alpha) {
  const int bh = blockIdx.y;
  const int nb = M / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int row0 = (blockIdx.x / nb) * 32 + (wave >> 1) * 16;
  const int col0 = (blockIdx.x % nb) * 32 + (wave & 1) * 16;
  const float* Pm = P + (size_t)bh * M * M;
  const float* Qm = Q + (size_t)bh * M * M;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    float x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 32 * ks + 8 * g + e;
      x[e] = Pm[(size_t)(row0 + c16) * M + k];
      const float qv = Qm[(size_t)k * M + col0 + c16];
      y[e] = beta != 0.f ? ((k == col0 + c16 ? beta : 0.f) - qv) : qv;
    }
    if constexpr (F32)
      acc = mma8_f32(x, y, acc);
    else
      acc = mma<3>(split8(x), split8(y), acc);
  }
  float* Cm = C + (size_t)bh * M * M;
#pragma unroll
  for (int r = 0; r < 4; ++r) Cm[(size_t)(row0 + 4 * g + r) * M + col0 + c16] = alpha * acc[r];
}

}  // namespace nys
