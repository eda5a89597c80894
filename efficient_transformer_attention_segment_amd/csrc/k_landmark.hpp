// Landmarks and the landmark Gram softmax.
//
// Pages: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.2
// (Q and K each scaled by d^-1/4), section 2.3 (segment means over n/m
// contiguous tokens), section 2.4 (A = softmax of the landmark products),
// section 2.5 (the init scale needs the column and row sums of A).
//
// k_landmark: one workgroup reduces `lpw` landmarks of one (batch, head)
// for both Q and K.  Each landmark's L rows are split over RS row slots of
// d / 8 threads (each thread owns 8 contiguous channels of a row), summed in
// float32 with eight rows in flight per thread, then the RS slots are folded
// in LDS in a fixed order (deterministic).  The scale d^-1/4 / L is applied
// once; the landmarks are written in float32 and as bf16 hi/lo operands.
//
// k_gram: one workgroup per head computes A = softmax(Qt Kt^T) and the
// head's maximum column sum and row sum of A.  For float32 I/O the products
// run on the float32 matrix core: A feeds the pseudo-inverse iteration, which
// magnifies an error in A by up to the condition number of A once it has
// converged, so A is formed in plain float32.  For bf16 I/O they are
// split-bf16 products (relative error about 2^-16).  The kernel boundary between the two is the
// only synchronisation (no device-wide fences).
#pragma once

#include "common.hpp"

namespace nys {

struct LandmarkArgs {
  int n, m, L, RS, lpw, BH, H;
  Strides in;           // of q and k
  int mr;               // landmarks of the method; m = mr rounded up to 32 (rows mr .. m-1 are zero)
  float scale;          // d^-1/4 / L
  float* qt;            // [BH][m][d] float32
  float* kt;
  __bf16* qt_hi;        // [BH][m][d] bf16 split of qt / kt
  __bf16* qt_lo;
  __bf16* kt_hi;
  __bf16* kt_lo;
  float* A;             // [BH][m][m]
  float* colmax;        // [BH]
  float* rowmax;        // [BH]
  unsigned long long* slots;  // [BH][2] pseudo-inverse blocks' tagged maxima, cleared by k_landmark
};

// Logits of padding landmark columns (16 ct + lane % 16 >= mr) -> -inf, in a
// row of C tiles acc[ct] (rows 4g + r, column lane % 16).
template <int TM>
__device__ __forceinline__ void pad_mask_cols(f32x4 (&acc)[TM], int mr) {
  const int c16 = threadIdx.x & 15;
#pragma unroll
  for (int ct = 0; ct < TM; ++ct)
    if (16 * ct + c16 >= mr) acc[ct] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
}

// LDS staging of Kt for the Gram (elements): bf16 hi / lo planes with row
// stride D + 8 (bf16 I/O) or float32 rows with stride D + 4 (float32 I/O).
template <int M, bool F32, int D>
constexpr int gram_kst_bytes() {
  return F32 ? M * (D + 4) * 4 : 2 * M * (D + 8) * 2;
}

// A = softmax(Qt Kt^T) for one head, by the NW waves of the block; writes A
// and the head's maximum column and row sums (also returned in wred[0] and
// wred[1] to every thread).  M: landmarks padded to a multiple of 32.  Kt comes into LDS (kst,
// gram_kst_bytes) in one coalesced pass first; each wave takes row tiles
// wave, wave + NW, ...  csum: LDS scratch of (M/16) * M floats; wred: 2 * NW.
template <int M, bool F32, int NW, int D>
__device__ void landmark_gram_tail(const LandmarkArgs& a, int bh, float* csum, float* wred, void* kst) {
  constexpr int TM = M / 16, DK = D / 32, KLD32 = D + 4, KLD16 = D + 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const float* qt = a.qt + (size_t)bh * M * D;
  float* A = a.A + (size_t)bh * M * M;
  float* const kf32 = reinterpret_cast<float*>(kst);
  __bf16* const kb16 = reinterpret_cast<__bf16*>(kst);
  if constexpr (F32) {
    const float4* kt = reinterpret_cast<const float4*>(a.kt + (size_t)bh * M * D);
    for (int i = threadIdx.x; i < M * (D / 4); i += 64 * NW)
      *reinterpret_cast<float4*>(kf32 + (i / (D / 4)) * KLD32 + 4 * (i % (D / 4))) = kt[i];
  } else {
    const uint4* kh = reinterpret_cast<const uint4*>(a.kt_hi + (size_t)bh * M * D);
    const uint4* kl = reinterpret_cast<const uint4*>(a.kt_lo + (size_t)bh * M * D);
    for (int i = threadIdx.x; i < M * (D / 8); i += 64 * NW) {
      *reinterpret_cast<uint4*>(kb16 + (i / (D / 8)) * KLD16 + 8 * (i % (D / 8))) = kh[i];
      *reinterpret_cast<uint4*>(kb16 + (M + i / (D / 8)) * KLD16 + 8 * (i % (D / 8))) = kl[i];
    }
  }
  __syncthreads();
  float rmax_w = 0.f;
  for (int rt = wave; rt < TM; rt += NW) {
    // operands: element e of lane (g, c16) is k = 32 ks + 8 g + e
    float ax[DK][8];
    Frag2 af[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const size_t off = (size_t)(rt * 16 + c16) * D + ks * 32 + g * 8;
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ax[ks][e] = qt[off + e];
      } else {
        af[ks].hi = *reinterpret_cast<const bf16x8*>(a.qt_hi + (size_t)bh * M * D + off);
        af[ks].lo = *reinterpret_cast<const bf16x8*>(a.qt_lo + (size_t)bh * M * D + off);
      }
    }
    f32x4 acc[TM];
#pragma unroll
    for (int ct = 0; ct < TM; ++ct) {
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const int row = ct * 16 + c16, col = ks * 32 + g * 8;
        if constexpr (F32) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = kf32[row * KLD32 + col + e];
          acc[ct] = mma8_f32(ax[ks], x, acc[ct]);
        } else {
          Frag2 bf;
          bf.hi = *reinterpret_cast<const bf16x8*>(kb16 + row * KLD16 + col);
          bf.lo = *reinterpret_cast<const bf16x8*>(kb16 + (M + row) * KLD16 + col);
          acc[ct] = mma<3>(af[ks], bf, acc[ct]);
        }
      }
    }
    // row softmax: row 16rt + 4g + r, columns spread over ct and lane & 15;
    // padding columns take no weight and padding rows are zero
    if (a.mr < M) pad_mask_cols(acc, a.mr);
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
      const float inv = rt * 16 + g * 4 + r < a.mr ? 1.0f / s : 0.f;
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
    for (int ct = 0; ct < TM; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) A[(size_t)(rt * 16 + g * 4 + r) * M + ct * 16 + c16] = acc[ct][r];
      // column partial sums over this row tile
      float cs = acc[ct][0] + acc[ct][1] + acc[ct][2] + acc[ct][3];
      cs = sum_g(cs);
      if (g == 0) csum[rt * M + ct * 16 + c16] = cs;
    }
  }
  rmax_w = max_g(rmax_w);
  if (lane == 0) wred[wave] = rmax_w;
  __syncthreads();
  // column sums in a fixed order, then the block maximum
  float cmax = 0.f;
  for (int j = threadIdx.x; j < M; j += 64 * NW) {
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
  if (threadIdx.x == 0) {
    a.rowmax[bh] = rm;
    a.colmax[bh] = cm;
    wred[0] = cm;
    wred[1] = rm;
  }
  __syncthreads();
}

// grid: (m / lpw, BH), block 256, with (D / 8) * RS * lpw == 256.
template <typename IO, int M, int D>
__global__ __launch_bounds__(256) void k_landmark(const IO* __restrict__ q, const IO* __restrict__ k,
                                                   LandmarkArgs a) {
  constexpr int CW = 8;          // channels per thread
  constexpr int TPR = D / CW;    // threads per row
  constexpr int UNR = 8;         // rows in flight per thread and tensor
  __shared__ float red[2][256][CW + 1];

  const int t = threadIdx.x;
  const int bh = blockIdx.y;
  const int RS = a.RS, lpw = a.lpw, L = a.L;
  const int c = t % TPR;
  const int rs = (t / TPR) % RS;
  const int j = t / (TPR * RS);
  const int i = blockIdx.x * lpw + j;
  const bool live = i < a.mr;  // padding landmarks stay zero
  const long long st = a.in.t;
  const long long base = a.in.base(bh, a.H) + (long long)(live ? i : 0) * L * st + c * CW;
  if (blockIdx.x == 0 && t < 2) a.slots[2 * blockIdx.y + t] = 0ull;  // written in the next launch

  float sq[CW], sk[CW];
#pragma unroll
  for (int e = 0; e < CW; ++e) sq[e] = sk[e] = 0.f;
  int r = live ? rs : L;
  for (; r + (UNR - 1) * RS < L; r += UNR * RS) {
    float xq[UNR][CW], xk[UNR][CW];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      IOTraits<IO>::load8(q + base + (r + u * RS) * st, xq[u]);
      IOTraits<IO>::load8(k + base + (r + u * RS) * st, xk[u]);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int e = 0; e < CW; ++e) {
        sq[e] += xq[u][e];
        sk[e] += xk[u][e];
      }
  }
  for (; r < L; r += RS) {
    float xq[CW], xk[CW];
    IOTraits<IO>::load8(q + base + r * st, xq);
    IOTraits<IO>::load8(k + base + r * st, xk);
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      sq[e] += xq[e];
      sk[e] += xk[e];
    }
  }
#pragma unroll
  for (int e = 0; e < CW; ++e) {
    red[0][t][e] = sq[e];
    red[1][t][e] = sk[e];
  }
  __syncthreads();
  for (int idx = t; idx < 2 * lpw * D; idx += 256) {
    const int which = idx / (lpw * D);
    const int rem = idx % (lpw * D);
    const int jj = rem / D, col = rem % D;
    const int cc = col / CW, e = col % CW;
    float s = 0.f;
    for (int q2 = 0; q2 < RS; ++q2) s += red[which][(jj * RS + q2) * TPR + cc][e];
    s *= a.scale;
    const size_t o = ((size_t)bh * a.m + blockIdx.x * lpw + jj) * D + col;
    __bf16 hi, lo;
    split1(s, hi, lo);
    if (which == 0) {
      a.qt[o] = s;
      a.qt_hi[o] = hi;
      a.qt_lo[o] = lo;
    } else {
      a.kt[o] = s;
      a.kt_hi[o] = hi;
      a.kt_lo[o] = lo;
    }
  }
}

// grid: BH, block 64 gram_waves<M>() threads, dynamic LDS gram_lds_bytes<M, F32>().
template <int M>
constexpr int gram_waves() {
  return M / 16 < 16 ? (M / 16 < 4 ? 4 : M / 16) : 16;
}
template <int M, bool F32, int D>
constexpr int gram_lds_bytes() {
  return gram_kst_bytes<M, F32, D>() + 4 * ((M / 16) * M + 2 * gram_waves<M>());
}
template <int M, bool F32, int D>
__global__ __launch_bounds__(64 * gram_waves<M>()) void k_gram(LandmarkArgs a) {
  extern __shared__ __align__(16) float gram_smem[];
  float* const csum = gram_smem + gram_kst_bytes<M, F32, D>() / 4;
  float* const wred = csum + (M / 16) * M;
  landmark_gram_tail<M, F32, gram_waves<M>(), D>(a, blockIdx.x, csum, wred, gram_smem);
}

}  // namespace nys
