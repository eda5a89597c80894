// Combine the per-chunk B V partials and form W = Z (B V).
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4:
// new_value = kernel_3 V and the context is the product of F A^+ with it;
// the product is taken here in the order F (Z (B V)), equal in exact
// arithmetic.
//
// k_merge merges 16 landmark rows per block over the S key chunks with the
// log-sum-exp rule (fixed chunk order, deterministic); a row whose chunks
// saw no valid key gives B V = 0.  k_w then forms W = Z (B V), 32 rows per
// block (float32 matrix-core products for float32 I/O, where a converged Z
// has large entries whose products cancel; split-bf16 products for bf16
// I/O), and writes W twice: float32
// row-major, and as the ready-made bf16 hi/lo A-operand fragments of W^T
// that the output kernel loads with one 16-byte read per lane (rows in the
// output kernel's channel order, k in the paired order).  Kernel boundaries order
// the three steps; there are no device-wide fences.
#pragma once

#include "common.hpp"
#include "k_conv.hpp"

namespace nys {

struct MergeArgs {
  const float* pmax;   // [BH][S][M], log2 units
  const float* psum;
  const float* pacc;   // [BH][S][M][64]
  const float* Z;      // [BH][M][M]
  float* BV;           // [BH][M][64]
  float* W;            // [BH][M][64]
  __bf16* wf_hi;       // [BH][4][M/32][64][8]
  __bf16* wf_lo;
  int S;
};

// grid (M/16, BH): B V rows [16 bx, 16 bx + 16).  Thread (row, 4-channel
// quad); the chunk loops are unrolled by 8 so the partial loads overlap.
template <int M>
__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  constexpr int U = 8;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int i = blockIdx.x * 16 + (t >> 4);
  const int d0 = (t & 15) * 4;
  const size_t base = (size_t)bh * a.S * M + i;  // row of chunk s: base + s * M
  float mx = NEG_BIG;
  int s = 0;
  for (; s + U <= a.S; s += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a.pmax[base + (size_t)(s + u) * M];
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, v[u]);
  }
  for (; s < a.S; ++s) mx = fmaxf(mx, a.pmax[base + (size_t)s * M]);
  float tot = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  s = 0;
  for (; s + U <= a.S; s += U) {
    float pm[U], ps[U];
    float4 pa[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t row = base + (size_t)(s + u) * M;
      pm[u] = a.pmax[row];
      ps[u] = a.psum[row];
      pa[u] = *reinterpret_cast<const float4*>(a.pacc + row * HD + d0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = fast_exp2(pm[u] - mx);
      tot += ps[u] * wgt;
      acc[0] += pa[u].x * wgt;
      acc[1] += pa[u].y * wgt;
      acc[2] += pa[u].z * wgt;
      acc[3] += pa[u].w * wgt;
    }
  }
  for (; s < a.S; ++s) {
    const size_t row = base + (size_t)s * M;
    const float wgt = fast_exp2(a.pmax[row] - mx);
    tot += a.psum[row] * wgt;
    const float4 p = *reinterpret_cast<const float4*>(a.pacc + row * HD + d0);
    acc[0] += p.x * wgt;
    acc[1] += p.y * wgt;
    acc[2] += p.z * wgt;
    acc[3] += p.w * wgt;
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  *reinterpret_cast<float4*>(a.BV + ((size_t)bh * M + i) * HD + d0) =
      make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
}

// grid (M/32, BH): W rows [32 bx, 32 bx + 32) = Z[rows, :] (B V), then the
// W^T fragments of k step bx for every d tile.
template <int M, bool B16, bool F32>
__global__ __launch_bounds__(256) void k_w(MergeArgs a) {
  constexpr int KS = M / 32;
  __shared__ float wt[32][HD + 1];
  const int bh = blockIdx.y, kb = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 4, c16 = lane & 15;
  const float* Z = a.Z + (size_t)bh * M * M;
  const float* BV = a.BV + (size_t)bh * M * HD;
  float* W = a.W + (size_t)bh * M * HD;
  // wave w: row tile (w >> 1) of the block, d tiles {2 (w & 1), 2 (w & 1) + 1}
  const int rt = 2 * kb + (wave >> 1);
#pragma unroll
  for (int dd = 0; dd < 2; ++dd) {
    const int dt = 2 * (wave & 1) + dd;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = Z[(size_t)(16 * rt + c16) * M + 32 * ks + 8 * g + e];
        y[e] = BV[(size_t)(32 * ks + 8 * g + e) * HD + 16 * dt + c16];
      }
      if constexpr (F32)
        acc = mma8_f32(x, y, acc);
      else
        acc = mma<3>(split8(x), split8(y), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (wave >> 1) + 4 * g + r;
      wt[row][16 * dt + c16] = acc[r];
      W[(size_t)(32 * kb + row) * HD + 16 * dt + c16] = acc[r];
    }
  }
  __syncthreads();
  // fragments (dt, kb, lane'): element e = W[32 kb + kp][dmap(dt, rho)]
  __bf16* wh = a.wf_hi + (size_t)bh * 4 * KS * 64 * 8;
  __bf16* wl = a.wf_lo + (size_t)bh * 4 * KS * 64 * 8;
  {
    const int dt = t >> 6, ln = t & 63;
    const int rho = ln & 15, gg = ln >> 4;
    const int d = dmap<B16>(dt, rho);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = wt[e < 4 ? 4 * gg + e : 16 + 4 * gg + e - 4][d];
    const Frag2 f = split8(x);
    const size_t ent = (size_t)(dt * KS + kb) * 64 + ln;
    *reinterpret_cast<bf16x8*>(wh + ent * 8) = f.hi;
    *reinterpret_cast<bf16x8*>(wl + ent * 8) = f.lo;
  }
}

}  // namespace nys
