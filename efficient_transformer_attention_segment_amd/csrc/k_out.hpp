// Output pass: out = F W + conv(V), with F = softmax(Qs Kt^T).
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4
// (kernel_1 F = softmax(Q against the key landmarks), n x m; the context is
// F times A^+ times B V) and section 2.6 (context += depthwise conv of V).
//
// A workgroup covers 128 tokens of one head (4 waves x 2 tiles of 16).  The
// key landmarks, the W^T fragments and a V window (tokens t0 - 32 .. t0 +
// 176) are staged in LDS once (bf16: by DMA, V read back transposed;
// float32: through registers as bf16 hi/lo with V stored transposed), with
// every wave's Q rows already loading as B fragments.  Per 16-token tile a
// wave:
//   forms S^T = Kt Q^T (m x 16) on the matrix cores,
//   takes the softmax down each column with the whole F row in registers
//   (m <= 256: no online rescaling needed),
//   accumulates O^T = W^T F^T, F used directly from the S^T C tiles,
//   adds the convolution as three banded Toeplitz products into the same
//   accumulators,
//   and stores 16 contiguous channels per lane.
// Qt / Kt carry the d^-1/4 factor, Q does not: logits get the other factor.
#pragma once

#include "common.hpp"
#include "k_conv.hpp"
#include "k_pinv.hpp"

namespace nys {

struct OutArgs {
  const void* q;
  const void* v;
  const __bf16* zero;    // >= 128 zero bytes (rows outside the sequence)
  const float* conv_w;   // [H][65] or null
  const __bf16* kt_hi;   // [BH][M][64]
  const __bf16* kt_lo;
  const __bf16* wf_hi;   // [BH][4][M/32][64][8]
  const __bf16* wf_lo;
  void* out;
  int n, H;
  float lscale;          // d^-1/4
};

constexpr int OUT_TOK = 128;                 // tokens per workgroup
constexpr int OUT_WIN = OUT_TOK + 80;        // V window rows (t0-32 .. t0+176)
constexpr int OUT_VWLD = OUT_WIN + 8;

template <typename IO, int M>
struct OutLayout {
  static constexpr int NS = IOTraits<IO>::NS;
  static constexpr int KS = M / 32;
  static constexpr int KLD = HD + 8;
  static constexpr int KT_ELEMS = M * KLD;                 // per part
  static constexpr int WF_ELEMS = 4 * KS * 64 * 8;         // per part
  static constexpr int V_ELEMS = HD * OUT_VWLD;            // per part
  static constexpr int PARTS = NS == 3 ? 2 : 1;
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_WF = OFF_KT + PARTS * KT_ELEMS;
  static constexpr int OFF_V = OFF_WF + PARTS * WF_ELEMS;
  static constexpr int TOTAL = OFF_V + PARTS * V_ELEMS;
  static constexpr int LDS_BYTES = TOTAL * 2;
};

// bf16 inputs: K~, the W^T fragments and the V window are copied into LDS
// by DMA (row-major, swizzled chunks; rows outside [0, n) from a zero page)
// and the V^T convolution operand is read back with transposed reads.
template <int M>
struct OutLayoutDMA {
  static constexpr int KS = M / 32;
  static constexpr int OFF_KT = 0;                        // M rows x 64
  static constexpr int OFF_WF = OFF_KT + M * HD;          // 4 KS 64 8
  static constexpr int OFF_V = OFF_WF + 4 * KS * 64 * 8;  // OUT_WIN rows x 64
  static constexpr int TOTAL = OFF_V + OUT_WIN * HD;
  static constexpr int LDS_BYTES = TOTAL * 2;
};

template <int M>
__device__ __forceinline__ void out_stage_dma(const OutArgs& a, int bh, int t0, __bf16* lds) {
  using Ly = OutLayoutDMA<M>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const u16* V = reinterpret_cast<const u16*>(a.v) + (size_t)bh * a.n * HD;
  const __bf16* kt = a.kt_hi + (size_t)bh * M * HD;
  const __bf16* wf = a.wf_hi + (size_t)bh * 4 * Ly::KS * 64 * 8;
  const int rsub = lane >> 3;
  // key landmarks: M / 8 copies of 8 rows
  for (int c = wave; c < M / 8; c += 4) {
    const int row = 8 * c + rsub;
    const int chunk = (lane & 7) ^ (row & 7);
    dma16(kt + (size_t)row * HD + 8 * chunk, lds + Ly::OFF_KT + 8 * c * HD);
  }
  // W^T fragments: contiguous, 1 KB per copy
  for (int c = wave; c < 4 * Ly::KS; c += 4) dma16(wf + (size_t)c * 512 + 8 * lane, lds + Ly::OFF_WF + 512 * c);
  if (a.conv_w != nullptr) {
    for (int c = wave; c < OUT_WIN / 8; c += 4) {
      const int row = 8 * c + rsub;
      const int chunk = (lane & 7) ^ (row & 7);
      const int s = t0 - HALO + row;
      const void* src = (s >= 0 && s < a.n) ? (const void*)(V + (size_t)s * HD + 8 * chunk) : (const void*)a.zero;
      dma16(src, lds + Ly::OFF_V + 8 * c * HD);
    }
  }
}

// Per-lane offsets of the transposed conv reads inside the DMA-staged
// window: for a tile at window row wc the read of (kk, half, dt) sits at
// (wc + 32 kk) * 64 + off[half][dt].  The swizzle term only depends on
// (row & 7), which wc (a multiple of 16) and 32 kk leave unchanged.
__device__ __forceinline__ void conv_dma_offsets(int (&off)[2][4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int row = 8 * g + (c16 >> 2) + 4 * half;
      const int c0 = dmap_run<true>(dt, c16 & 3);
      off[half][dt] = row * HD + 8 * ((c0 >> 3) ^ (row & 7)) + (c0 & 7);
    }
}

// Convolution for one 16-token tile from the DMA-staged window (bf16 V is
// exact, taps split hi + lo).
__device__ __forceinline__ void conv_tile_dma(const __bf16* vw, int wc, const int (&off)[2][4], const Frag2 (&tap)[3],
                                              f32x4 (&oacc)[4]) {
  const __bf16* base = vw + wc * HD;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x4 x0 = lds_read_tr(base + 32 * kk * HD + off[0][dt]);
      const bf16x4 x1 = lds_read_tr(base + 32 * kk * HD + off[1][dt]);
      const bf16x8 vh = cat44(x0, x1);
      oacc[dt] = mfma(vh, tap[kk].hi, oacc[dt]);
      oacc[dt] = mfma(vh, tap[kk].lo, oacc[dt]);
    }
  }
}

template <typename IO, int M>
__global__ __launch_bounds__(256) void k_out(OutArgs a) {
  extern __shared__ __align__(16) __bf16 lds_dyn[];
  using Ly = OutLayout<IO, M>;
  constexpr int NS = Ly::NS, KS = Ly::KS, TM = M / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, h = bh % a.H;
  const int t0 = blockIdx.x * OUT_TOK;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * HD;
  const IO* V = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * HD;

  __bf16* kth = lds_dyn + Ly::OFF_KT;
  __bf16* ktl = kth + Ly::KT_ELEMS;
  __bf16* wfh = lds_dyn + Ly::OFF_WF;
  __bf16* wfl = wfh + Ly::WF_ELEMS;
  __bf16* vh = lds_dyn + Ly::OFF_V;
  __bf16* vl = vh + Ly::V_ELEMS;

  constexpr bool DMA = sizeof(IO) == 2;
  using LyD = OutLayoutDMA<M>;
  // ---- stage Kt, W^T fragments and the V window
  if constexpr (DMA) {
    out_stage_dma<M>(a, bh, t0, lds_dyn);
  } else {
    const __bf16* src_h = a.kt_hi + (size_t)bh * M * HD;
    const __bf16* src_l = a.kt_lo + (size_t)bh * M * HD;
    for (int idx = threadIdx.x; idx < M * 8; idx += 256) {
      const int row = idx >> 3, cc = idx & 7;
      *reinterpret_cast<bf16x8*>(kth + row * Ly::KLD + 8 * cc) =
          *reinterpret_cast<const bf16x8*>(src_h + (size_t)row * HD + 8 * cc);
      if constexpr (NS == 3)
        *reinterpret_cast<bf16x8*>(ktl + row * Ly::KLD + 8 * cc) =
            *reinterpret_cast<const bf16x8*>(src_l + (size_t)row * HD + 8 * cc);
    }
    const __bf16* wsh = a.wf_hi + (size_t)bh * Ly::WF_ELEMS;
    const __bf16* wsl = a.wf_lo + (size_t)bh * Ly::WF_ELEMS;
    for (int idx = threadIdx.x; idx < Ly::WF_ELEMS / 8; idx += 256) {
      *reinterpret_cast<bf16x8*>(wfh + 8 * idx) = *reinterpret_cast<const bf16x8*>(wsh + 8 * idx);
      if constexpr (NS == 3)
        *reinterpret_cast<bf16x8*>(wfl + 8 * idx) = *reinterpret_cast<const bf16x8*>(wsl + 8 * idx);
    }
    if (a.conv_w != nullptr) stage_v_window<IO>(V, a.n, t0, OUT_WIN, vh, vl, OUT_VWLD);
  }
  // Q B fragments of both tiles, in flight with the staging copies
  Frag2 qf2[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;
    const int tok = min(ts + c16, a.n - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (DMA) {
        qf2[u][ks].hi = *reinterpret_cast<const bf16x8*>(Q + (size_t)tok * HD + 32 * ks + 8 * g);
      } else {
        float x[8];
        IOTraits<IO>::load8(Q + (size_t)tok * HD + 32 * ks + 8 * g, x);
        qf2[u][ks] = make_frag<NS>(x);
      }
    }
  }
  int coff[2][4];
  if constexpr (DMA) conv_dma_offsets(coff);
  Frag2 tap[3];
  if (a.conv_w != nullptr) conv_taps(a.conv_w + (size_t)h * TAPS, tap);
  if constexpr (DMA) {
    wait_vmcnt<0>();
    barrier_only();
  } else {
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;  // tile start
    if (ts >= a.n) continue;
    const int tok = ts + c16;
    const Frag2(&qf)[2] = qf2[u];
    // S^T = Kt Q^T: sacc[it][r] = logit(tok, landmark 16 it + 4g + r)
    f32x4 sacc[TM];
#pragma unroll
    for (int it = 0; it < TM; ++it) {
      sacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag2 kf;
        if constexpr (DMA) {
          kf.hi = *reinterpret_cast<const bf16x8*>(lds_dyn + LyD::OFF_KT + swz(16 * it + c16, 4 * ks + g));
        } else {
          const int off = (16 * it + c16) * Ly::KLD + 32 * ks + 8 * g;
          kf.hi = *reinterpret_cast<const bf16x8*>(kth + off);
          if constexpr (NS == 3) kf.lo = *reinterpret_cast<const bf16x8*>(ktl + off);
        }
        sacc[it] = mma<NS>(kf, qf[ks], sacc[it]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[it][r]);
    mx = max_g(mx);
    const float ls2 = a.lscale * LOG2E;
    const float mb = mx * ls2;
    float sum = 0.f;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(sacc[it][r], ls2, -mb));
        sacc[it][r] = p;
        sum += p;
      }
    sum = sum_g(sum);
    const float inv = 1.0f / sum;
    // O^T = W^T F^T
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8] = {sacc[2 * ks][0] * inv,     sacc[2 * ks][1] * inv,     sacc[2 * ks][2] * inv,
                    sacc[2 * ks][3] * inv,     sacc[2 * ks + 1][0] * inv, sacc[2 * ks + 1][1] * inv,
                    sacc[2 * ks + 1][2] * inv, sacc[2 * ks + 1][3] * inv};
      const Frag2 pf = make_frag<NS>(x);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        Frag2 wf;
        const int off = ((dt * KS + ks) * 64 + lane) * 8;
        if constexpr (DMA) {
          wf.hi = *reinterpret_cast<const bf16x8*>(lds_dyn + LyD::OFF_WF + off);
        } else {
          wf.hi = *reinterpret_cast<const bf16x8*>(wfh + off);
          if constexpr (NS == 3) wf.lo = *reinterpret_cast<const bf16x8*>(wfl + off);
        }
        oacc[dt] = mma<NS>(wf, pf, oacc[dt]);
      }
    }
    if (a.conv_w != nullptr) {
      if constexpr (DMA)
        conv_tile_dma(lds_dyn + LyD::OFF_V, ts - t0, coff, tap, oacc);
      else
        conv_tile<NS, DMA>(vh, vl, OUT_VWLD, ts - t0, tap, oacc);
    }
    store_row16<IO, DMA>(reinterpret_cast<IO*>(a.out) + ((size_t)bh * a.n + tok) * HD, oacc);
  }
}

}  // namespace nys
