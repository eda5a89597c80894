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
// [0, n) are zero.
template <typename IO, int D = HD>
__device__ void stage_v_window(const IO* __restrict__ V, long long st, int n, int t0, int win, __bf16* Vh, __bf16* Vl,
                               int ld) {
  constexpr int NS = IOTraits<IO>::NS, CPR = D / 8;
  for (int idx = threadIdx.x; idx < win * CPR; idx += blockDim.x) {
    const int row = idx / CPR, cc = idx % CPR;
    const int s = t0 - HALO + row;
    float x[8];
    if (s >= 0 && s < n) {
      IOTraits<IO>::load8(V + s * st + 8 * cc, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split1(x[e], h, l);
      Vh[(8 * cc + e) * ld + row] = h;
      if constexpr (NS == 3) Vl[(8 * cc + e) * ld + row] = l;
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
