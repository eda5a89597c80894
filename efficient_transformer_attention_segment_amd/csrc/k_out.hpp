// Output pass: out = F W + conv(V), with F = softmax(Qs Kt^T).
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4
// (kernel_1 F = softmax(Q against the key landmarks), n x m; the context is
// F times A^+ times B V) and section 2.6 (context += depthwise conv of V).
//
// A workgroup covers 128 tokens of one head (4 waves x 2 tiles of 16).  The
// key landmarks (bf16 hi/lo), the W^T fragments and a transposed V window
// (tokens t0 - 32 .. t0 + 176) are staged in LDS once.  Per 16-token tile a
// wave:
//   loads its Q rows straight from HBM as B fragments (16 bytes per lane),
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

  // ---- stage Kt, W^T fragments and the V window
  {
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
  Frag2 tap[3];
  if (a.conv_w != nullptr) conv_taps(a.conv_w + (size_t)h * TAPS, tap);
  __syncthreads();

#pragma unroll 1
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;  // tile start
    if (ts >= a.n) break;
    const int tok = ts + c16;
    // Q B fragments
    Frag2 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float x[8];
      IOTraits<IO>::load8(Q + (size_t)tok * HD + 32 * ks + 8 * g, x);
      qf[ks] = make_frag<NS>(x);
    }
    // S^T = Kt Q^T: sacc[it][r] = logit(tok, landmark 16 it + 4g + r)
    f32x4 sacc[TM];
#pragma unroll
    for (int it = 0; it < TM; ++it) {
      sacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag2 kf;
        const int off = (16 * it + c16) * Ly::KLD + 32 * ks + 8 * g;
        kf.hi = *reinterpret_cast<const bf16x8*>(kth + off);
        if constexpr (NS == 3) kf.lo = *reinterpret_cast<const bf16x8*>(ktl + off);
        sacc[it] = mma<NS>(kf, qf[ks], sacc[it]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sacc[it][r] *= a.lscale;
        mx = fmaxf(mx, sacc[it][r]);
      }
    mx = max_g(mx);
    float sum = 0.f;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2((sacc[it][r] - mx) * LOG2E);
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
        wf.hi = *reinterpret_cast<const bf16x8*>(wfh + off);
        if constexpr (NS == 3) wf.lo = *reinterpret_cast<const bf16x8*>(wfl + off);
        oacc[dt] = mma<NS>(wf, pf, oacc[dt]);
      }
    }
    if (a.conv_w != nullptr) conv_tile<NS>(vh, vl, OUT_VWLD, ts - t0, tap, oacc);
    float vals[16];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) vals[4 * dt + r] = oacc[dt][r];
    IOTraits<IO>::store16(reinterpret_cast<IO*>(a.out) + ((size_t)bh * a.n + tok) * HD + 16 * g, vals);
  }
}

}  // namespace nys
