// Combine the per-chunk B V partials and form W = Z (B V), in one launch.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4:
// new_value = kernel_3 V and the context is the product of F A^+ with it;
// the product is taken here in the order F (Z (B V)), equal in exact
// arithmetic.
//
// Both steps are independent per output channel, so a workgroup owns one
// 4-channel run of one head and needs nothing from the others:
//   1. merge: B V[:, run] over the S key chunks with the log-sum-exp rule
//      (each thread folds a fixed subset of chunks for one landmark row,
//      then the subsets are folded in a fixed order: deterministic).  A row
//      whose chunks saw no valid key gives B V = 0;
//   2. W[:, run] = Z B V[:, run] as float32 dot products (each thread a
//      fixed slice of k for one row, slices summed in a fixed order);
//   3. the run's part of the W^T A-operand fragments (bf16 hi/lo) that the
//      output pass loads with one 16-byte read per lane: rows in the output
//      pass's channel order, k in the paired order.
// B V and W are also written float32 row-major.  The partial sums are
// stored run-major ([chunk][run][row][4]), so a wave's loads are contiguous.
// The d / 4 workgroups of a head are placed on one XCD (block i runs on XCD
// i mod 8), so the per-row maxima and sums that all of them read are fetched
// into one L2 only.
#pragma once

#include "common.hpp"
#include "k_conv.hpp"

namespace nys {

struct MergeArgs {
  const float* pmax;   // [BH][S][M], log2 units
  const float* psum;
  const float* pacc;   // [BH][S][d/4][M][4]: 4-channel runs, each run's rows contiguous
  const float* Z;      // [BH][M][M]
  float* BV;           // [BH][M][d]
  float* W;            // [BH][M][d]
  __bf16* wf_hi;       // [BH][d/16][M/32][64][8]
  __bf16* wf_lo;
  float* lse;          // [BH][M] or null: log2 of each B row's normaliser (+inf for a row with no kept key)
  int S, BH;
};

// Grid size for BH heads of D channels: D / 4 runs per head, heads in
// groups of 8 (one per XCD); blocks of a missing head return at once.
inline int mw_blocks(int BH, int D) { return (D / 4) * 8 * ((BH + 7) / 8); }

// (head, run) of block id (id % 8 is the block's XCD)
template <int D>
__device__ __forceinline__ void mw_role(int id, int& bh, int& run) {
  constexpr int RUNS = D / 4;
  const int xcd = id & 7, slot = id >> 3;
  bh = 8 * (slot / RUNS) + xcd;
  run = slot % RUNS;
}

// k slices per row for the W step: the most (up to NT / M) that split the
// row into equal runs of a multiple of 4
template <int M, int NT>
constexpr int mw_ksp() {
  int k = NT / M;
  while (k > 1 && M % (4 * k) != 0) --k;
  return k;
}

template <int M, int NT>
struct MwLayout {
  static constexpr int SP = NT / M;            // chunk subsets per row
  static constexpr int KSP = mw_ksp<M, NT>();  // k slices per row
  static constexpr int KPER = M / KSP;         // k per slice
  static_assert(SP >= 1 && KPER % 4 == 0 && KPER * KSP == M, "landmark count");
  // float offsets in the block's scratch
  static constexpr int PART = 0;                      // [SP][M][6]: max, sum, 4 channels
  static constexpr int BVS = PART + SP * M * 6;       // [M][4]
  static constexpr int WPART = BVS + 4 * M;           // [KSP][M][4]
  static constexpr int WT = WPART + 4 * KSP * M;      // [M][5]
  static constexpr int FLOATS = WT + 5 * M;
};

// One (head, 4-channel run): merge, W and fragments (see the top of the
// file), by a block of NT threads.
template <int M, bool B16, int NT, int D>
__device__ void mw_body(const MergeArgs& a, int bh, int run, float* L) {
  static_assert(!B16 || D == 64, "the bf16 channel order is defined for d = 64");
  using Ly = MwLayout<M, NT>;
  constexpr int SP = Ly::SP, KSP = Ly::KSP, KPER = Ly::KPER, KS = M / 32;
  float* const part = L + Ly::PART;
  float4* const bvs = reinterpret_cast<float4*>(L + Ly::BVS);
  float4* const wpart = reinterpret_cast<float4*>(L + Ly::WPART);
  float* const wt = L + Ly::WT;
  const int dt = run >> 2, ra = run & 3;
  const int ch = dmap<B16>(dt, 4 * ra);  // channels ch .. ch + 3
  const int t = threadIdx.x;

  // this thread's first slice of its Z row, issued before the merge so its
  // latency overlaps the partial loads
  constexpr int ZPRE = KPER < 32 ? KPER : 32;
  const int zi = t % M, zs = t / M;
  const float* zrow = a.Z + ((size_t)bh * M + zi) * M + zs * KPER;
  float4 zpre[ZPRE / 4];
  if (zs < KSP) {
#pragma unroll
    for (int j = 0; j < ZPRE / 4; ++j) zpre[j] = *reinterpret_cast<const float4*>(zrow + 4 * j);
  }

  // 1. merge: row i, chunks sp, sp + SP, ...
  if (t < SP * M) {
    constexpr int U = 8;
    const int i = t % M, sp = t / M;
    const size_t base = (size_t)bh * a.S * M + i;  // row i of chunk s: base + s * M
    float mx = NEG_BIG, tot = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sp; s0 < a.S; s0 += U * SP) {
      float pm[U], ps[U], pa[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u * SP;
        if (s < a.S) {
          const size_t row = base + (size_t)s * M;
          pm[u] = a.pmax[row];
          ps[u] = a.psum[row];
          const float4 v =
              *reinterpret_cast<const float4*>(a.pacc + ((row - i) * (D / 4) + (size_t)(ch >> 2) * M + i) * 4);
          pa[u][0] = v.x;
          pa[u][1] = v.y;
          pa[u][2] = v.z;
          pa[u][3] = v.w;
        } else {
          pm[u] = NEG_BIG;
          ps[u] = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) pa[u][c] = 0.f;
        }
      }
      float bm = mx;
#pragma unroll
      for (int u = 0; u < U; ++u) bm = fmaxf(bm, pm[u]);
      const float a0 = fast_exp2(mx - bm);
      tot *= a0;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] *= a0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wgt = fast_exp2(pm[u] - bm);
        tot += ps[u] * wgt;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += pa[u][c] * wgt;
      }
      mx = bm;
    }
    float* pp = part + (sp * M + i) * 6;
    pp[0] = mx;
    pp[1] = tot;
#pragma unroll
    for (int c = 0; c < 4; ++c) pp[2 + c] = acc[c];
  }
  __syncthreads();
  if (t < M) {
    float mx = NEG_BIG;
#pragma unroll
    for (int sp = 0; sp < SP; ++sp) mx = fmaxf(mx, part[(sp * M + t) * 6]);
    float tot = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < SP; ++sp) {
      const float* pp = part + (sp * M + t) * 6;
      const float wgt = fast_exp2(pp[0] - mx);
      tot += pp[1] * wgt;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += pp[2 + c] * wgt;
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    if (a.lse != nullptr && run == 0) a.lse[(size_t)bh * M + t] = tot > 0.f ? mx + log2f(tot) : INFINITY;
    const float4 bv = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    bvs[t] = bv;
    *reinterpret_cast<float4*>(a.BV + ((size_t)bh * M + t) * D + ch) = bv;
  }
  __syncthreads();

  // 2. W[i, run] = sum_k Z[i, k] BV[k, run]: slice zs of row zi
  if (zs < KSP) {
    const int k0 = zs * KPER;
    float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < ZPRE / 4; ++j) {
      const float z[4] = {zpre[j].x, zpre[j].y, zpre[j].z, zpre[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 b = bvs[k0 + 4 * j + e];
        w[0] += z[e] * b.x;
        w[1] += z[e] * b.y;
        w[2] += z[e] * b.z;
        w[3] += z[e] * b.w;
      }
    }
#pragma unroll 8
    for (int kk = ZPRE; kk < KPER; kk += 4) {
      const float4 zz = *reinterpret_cast<const float4*>(zrow + kk);
      const float z[4] = {zz.x, zz.y, zz.z, zz.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 b = bvs[k0 + kk + e];
        w[0] += z[e] * b.x;
        w[1] += z[e] * b.y;
        w[2] += z[e] * b.z;
        w[3] += z[e] * b.w;
      }
    }
    wpart[zs * M + zi] = make_float4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();
  if (t < M) {
    float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSP; ++s) {
      const float4 p = wpart[s * M + t];
      w[0] += p.x;
      w[1] += p.y;
      w[2] += p.z;
      w[3] += p.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) wt[t * 5 + c] = w[c];
    *reinterpret_cast<float4*>(a.W + ((size_t)bh * M + t) * D + ch) = make_float4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();

  // 3. fragments (dt, kb, lane) for the lanes whose channel is in this run:
  // lane = 16 gg + 4 ra + b holds W[32 kb + kp][ch + b] with kp in the
  // paired order (4 gg .. 4 gg + 3, then 16 + 4 gg .. 16 + 4 gg + 3)
  if (t < KS * 16) {
    const int kb = t >> 4, gg = (t >> 2) & 3, b = t & 3;
    const int ln = 16 * gg + 4 * ra + b;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = wt[(32 * kb + (e < 4 ? 4 * gg + e : 16 + 4 * gg + e - 4)) * 5 + b];
    const Frag2 f = split8(x);
    const size_t ent = ((size_t)bh * (D / 16) * KS + (size_t)dt * KS + kb) * 64 + ln;
    *reinterpret_cast<bf16x8*>(a.wf_hi + ent * 8) = f.hi;
    // the bf16 output pass multiplies by W^T in one bf16 pass (its hi plane)
    if constexpr (!B16) *reinterpret_cast<bf16x8*>(a.wf_lo + ent * 8) = f.lo;
  }
}

// grid mw_blocks(BH) x NT: NT = M x (chunk subsets per row), chosen by the
// host so each thread folds at most one batch of 8 chunks where it can.
template <int M, bool B16, int NT, int D>
__global__ __launch_bounds__(NT) void k_mw(MergeArgs a) {
  __shared__ float L[MwLayout<M, NT>::FLOATS];
  int bh, run;
  mw_role<D>(blockIdx.x, bh, run);
  if (bh >= a.BH) return;
  mw_body<M, B16, NT, D>(a, bh, run, L);
}

}  // namespace nys
