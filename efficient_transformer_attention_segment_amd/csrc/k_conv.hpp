// Depthwise 65-tap 'same' convolution of V on the matrix cores.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.6: a
// per-head depthwise convolution along the sequence (kernel (65, 1),
// padding 32, no bias) applied to V and added to the attention output.
// Read as a cross-correlation: out[t] = sum_j w[h][j] V[t + j - 32], V = 0
// outside [0, n).
//
// For a tile of 16 output tokens the convolution is the banded (Toeplitz)
// product O^T[d][t] += sum_s V^T[d][s] T[s][t] with T[s][t] = w[s - t + 32],
// over the 80 positions s in [t0 - 32, t0 + 48), run as three 32-deep
// bf16 matrix-core steps that accumulate into the attention output's own C
// tiles.  V is staged in LDS transposed (position-contiguous per d row);
// the Toeplitz operand depends only on (s - t) so each lane builds its three
// fragments once per head.  Taps are split hi + lo; V is split too for
// float32 I/O.
#pragma once

#include "common.hpp"

namespace nys {

// Channel order of the output C tiles.  Row rho of d tile dt holds channel
// dmap<B16>(dt, rho); lane (t, g) holds rows 4g .. 4g+3 of the four d tiles.
//   B16 = false (natural): channel 16 dt + rho; lane g owns 16 dt + 4g + r,
//     so one 16-byte float32 store per d tile covers 64 contiguous bytes of
//     the row across the four lane groups.
//   B16 = true: channel 32 (dt / 2) + 8 (rho / 4) + 4 (dt % 2) + rho % 4; lane
//     g owns 8g .. 8g+7 and 32 + 8g .. 32 + 8g+7, so each 16-byte bf16 store
//     again covers 64 contiguous bytes.
// Either way a 4-channel run starts at a multiple of 4, which the
// transposed LDS reads need.
template <bool B16>
__device__ __forceinline__ int dmap(int dt, int rho) {
  if constexpr (B16) return 32 * (dt >> 1) + 8 * (rho >> 2) + 4 * (dt & 1) + (rho & 3);
  return 16 * dt + rho;
}
// First channel of the 4-run that lanes with (j % 4) == a address in a
// transposed read for d tile dt.
template <bool B16>
__device__ __forceinline__ int dmap_run(int dt, int a) {
  return dmap<B16>(dt, 4 * a);
}

// Store the lane's D / 4 output channels of one token row (B16 order only
// for D = 64); NT: nontemporal stores (final outputs nothing reads back).
template <typename IO, bool B16, int D = HD, bool NT = false>
__device__ __forceinline__ void store_row16(IO* row, const f32x4 (&acc)[D / 16]) {
  static_assert(!B16 || D == 64, "the bf16 channel order is defined for d = 64");
  const int g = (threadIdx.x & 63) >> 4;
  if constexpr (sizeof(IO) == 4) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float* const p = reinterpret_cast<float*>(row) + dmap<B16>(dt, 4 * g);
      if constexpr (NT)
        st_nt<f32x4>(p, acc[dt]);
      else
        *reinterpret_cast<float4*>(p) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    }
  } else if constexpr (B16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 2; ++r) w[2 * b + r] = pack_bf16x2(acc[2 * h + b][2 * r], acc[2 * h + b][2 * r + 1]);
      u16* const p = reinterpret_cast<u16*>(row) + 32 * h + 8 * g;
      if constexpr (NT)
        st_nt<u32x4>(p, u32x4{w[0], w[1], w[2], w[3]});
      else
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint32_t w0 = pack_bf16x2(acc[dt][0], acc[dt][1]);
      const uint32_t w1 = pack_bf16x2(acc[dt][2], acc[dt][3]);
      u16* const p = reinterpret_cast<u16*>(row) + 16 * dt + 4 * g;
      if constexpr (NT)
        st_nt<u32x2>(p, u32x2{w0, w1});
      else
        *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
    }
  }
}

// Stage V rows [t0 - 32, t0 - 32 + win) of one head (D channels),
// transposed, into Vh[d * ld + row] (and Vl when split).  Rows outside
// [0, n) are zero.  win and ld are even.  A thread takes two consecutive
// rows of four channels and stores each channel's two rows as one 4-byte
// word; a wave's 64 items are 16 row pairs x 4 channel groups, so at the
// row strides used here (4 channels apart, 4 ld / 2 words, an odd multiple
// of 16 banks) one store of the wave writes 64 distinct banks.  (Storing one
// row's 2-byte elements at a time put eight channels on the same banks.)
template <typename IO, int D = HD>
__device__ void stage_v_window(const IO* __restrict__ V, long long st, int n, int t0, int win, __bf16* Vh, __bf16* Vl,
                               int ld) {
  constexpr int NS = IOTraits<IO>::NS, GB = D / 16;  // blocks of four 4-channel groups
  const int pairs = win / 2;
  const int items = ((pairs + 15) / 16) * GB * 64;
  uint32_t* const wh = reinterpret_cast<uint32_t*>(Vh);
  uint32_t* const wl = reinterpret_cast<uint32_t*>(Vl);
  const int ldw = ld / 2;  // row stride in words
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int blk = it >> 6, l = it & 63;
    const int p = 16 * (blk / GB) + (l & 15), cg = 4 * (blk % GB) + (l >> 4);
    if (p >= pairs) continue;
    float x[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int s = t0 - HALO + 2 * p + r;
      if (s >= 0 && s < n) {
        if constexpr (sizeof(IO) == 4) {
          const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(V) + s * st + 4 * cg);
          x[r][0] = v.x;
          x[r][1] = v.y;
          x[r][2] = v.z;
          x[r][3] = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const u16*>(V) + s * st + 4 * cg);
          x[r][0] = __uint_as_float(v.x << 16);
          x[r][1] = __uint_as_float(v.x & 0xffff0000u);
          x[r][2] = __uint_as_float(v.y << 16);
          x[r][3] = __uint_as_float(v.y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[r][e] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h0, l0, h1, l1;
      split1(x[0][e], h0, l0);
      split1(x[1][e], h1, l1);
      const int w = (4 * cg + e) * ldw + p;  // rows 2p, 2p + 1 of channel 4 cg + e
      wh[w] = (uint32_t)__builtin_bit_cast(u16, h0) | ((uint32_t)__builtin_bit_cast(u16, h1) << 16);
      if constexpr (NS == 3)
        wl[w] = (uint32_t)__builtin_bit_cast(u16, l0) | ((uint32_t)__builtin_bit_cast(u16, l1) << 16);
    }
  }
}

// The three Toeplitz B fragments of this lane for head weights w[0..K-1],
// K odd, 1 <= K <= 65: window offset j (token t + j - 32) takes tap
// j - 32 + K / 2, zero outside [0, K); K = 65 is the pages' default.
__device__ __forceinline__ void conv_taps(const float* __restrict__ w, int K, Frag2 (&tap)[3]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int shift = K / 2 - HALO;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 32 * kk + 8 * g + e - c16 + shift;
      x[e] = (j >= 0 && j < K) ? w[j] : 0.f;
    }
    tap[kk] = split8(x);
  }
}

// oacc[dt] += conv for the 16-token tile starting at token ts, with the
// window staged from t0 - 32: wc = ts - t0 (window row of position ts - 32).
// Reads window rows [wc, wc + 96); the taps beyond the 80 needed are zero.
template <int NSV, bool B16, int D = HD>
__device__ __forceinline__ void conv_tile(const __bf16* Vh, const __bf16* Vl, int ld, int wc, const Frag2 (&tap)[3],
                                          f32x4 (&oacc)[D / 16]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int base = dmap<B16>(dt, c16) * ld + wc + 32 * kk + 8 * g;
      const bf16x8 vh = *reinterpret_cast<const bf16x8*>(Vh + base);
      oacc[dt] = mfma(vh, tap[kk].hi, oacc[dt]);
      oacc[dt] = mfma(vh, tap[kk].lo, oacc[dt]);
      if constexpr (NSV == 3) {
        const bf16x8 vl = *reinterpret_cast<const bf16x8*>(Vl + base);
        oacc[dt] = mfma(vl, tap[kk].hi, oacc[dt]);
      }
    }
  }
}

}  // namespace nys
