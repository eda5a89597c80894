// Attention weights on request (output_attentions).
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4
// (attention_probs = kernel_1 times the iterative inverse of kernel_2, an
// n x m matrix whose rows are the approximate attention weights), sections
// 2.7 and 5.3 (output_attentions hands those weights back; the full n x n
// softmax when the exact branch runs) and section 2.1 (the exact branch).
//
// k_probs (Nystrom path): P = F Z for 128 tokens x 64 landmark columns per
// workgroup.  The key landmarks (bf16 hi/lo as the output pass uses them;
// from L2 when LDS cannot hold them) and the Z^T operand fragments of the workgroup's 64 columns (split hi/lo
// from the float32 iterate) are staged in LDS.  Per 16-token tile a wave
// forms S^T = Kt Q^T, the softmax down each column with the whole F row in
// registers, and P^T = Z^T F^T with F taken straight from the S^T C tiles
// (float32-accurate split products: Z has large entries of both signs, so
// rounding it to bf16 would not do).  A lane then holds 4 consecutive
// columns of one token's row.  Above 64 landmarks the column blocks of one
// token block run on one XCD, so their Q reads meet in its L2.
//
// k_exact_probs (m == n): a wave owns 64 query rows (32 at d = 128); pass 1
// streams the keys for each row's maximum and sum, pass 2 recomputes the
// logits and writes the normalised weights, 16 keys per step.  Masked keys get 0; a row with
// no kept key is all zeros.
#pragma once

#include <algorithm>

#include "common.hpp"
#include "k_out.hpp"

namespace nys {

struct ProbsArgs {
  const void* q;            // [B,H,n,d] view, strides `in`
  const void* k;            // exact branch
  const uint8_t* key_mask;  // [B][n] or null (exact branch)
  const __bf16* kt_hi;      // [BH][M][d]
  const __bf16* kt_lo;
  const float* Z;           // [BH][M][M]
  void* probs;              // [BH][n][ldp], dense
  int n, H;
  int mr;                   // columns written: landmarks of the method (n when exact)
  int ldp;                  // row length of probs
  int grp;                  // token groups of PROBS_TOK per workgroup (Nystrom path)
  float lscale;             // logit factor (d^-1/4 against Kt, d^-1/2 exact)
  Strides in;
};

constexpr int PROBS_TOK = 128;  // tokens per group (4 waves x 2 tiles)
constexpr int PROBS_GRP_MAX = 8;  // token groups per workgroup at most

// Token groups per workgroup (the staged Kt and Z serve all of them): as
// many as keep about three workgroups per CU (768 on 256 CUs), at most
// PROBS_GRP_MAX.  Measured: two groups at 4 x 12 x 4096 (one or four were
// slower), four or more at 1 x 4 x 65536.
inline int probs_groups(int n, int BH, int ncb) {
  const long long blocks = (long long)((n + PROBS_TOK - 1) / PROBS_TOK) * BH * ncb;
  return (int)std::max(1LL, std::min((long long)PROBS_GRP_MAX, blocks / 768));
}
constexpr int PROBS_CB = 64;    // landmark columns per workgroup

template <typename IO, int M, int D>
struct ProbsLayout {
  static constexpr int NS = IOTraits<IO>::NS;
  static constexpr int KS = M / 32;
  static constexpr int KLD = D + 8;
  static constexpr int KT_ELEMS = M * KLD;               // per part
  static constexpr int ZF_ELEMS = 4 * KS * 64 * 8;       // per part: 4 column tiles x KS k-steps
  static constexpr int KPARTS = NS == 3 ? 2 : 1;
  // the key landmarks stay in L2 where LDS cannot hold them beside Z
  static constexpr bool KT_LDS = 2 * (KPARTS * KT_ELEMS + 2 * ZF_ELEMS) <= 160 * 1024;
  static constexpr int OFF_ZF = KT_LDS ? KPARTS * KT_ELEMS : 0;
  static constexpr int LDS_BYTES = 2 * (OFF_ZF + 2 * ZF_ELEMS);
  static constexpr int NCB = (M + PROBS_CB - 1) / PROBS_CB;
  static_assert(LDS_BYTES <= 160 * 1024, "k_probs LDS");
};

// Four consecutive weights of one row: one vector store when the row length
// keeps it aligned and all four columns exist, else element by element.
template <typename IO>
__device__ __forceinline__ void store_probs4(IO* row, int col, int ncol, bool vec, const f32x4& p) {
  if (vec && col + 3 < ncol) {
    if constexpr (sizeof(IO) == 4) {
      *reinterpret_cast<float4*>(row + col) = make_float4(p[0], p[1], p[2], p[3]);
    } else {
      *reinterpret_cast<uint2*>(row + col) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (col + r < ncol) {
        if constexpr (sizeof(IO) == 4)
          row[col + r] = p[r];
        else
          row[col + r] = f32_to_bf16u(p[r]);
      }
  }
}

// grid: (ceil(ceil(n / (128 grp)) / 8) * 8 * NCB, BH), block 256, dynamic LDS
// ProbsLayout<IO, M, D>::LDS_BYTES.
template <typename IO, int M, bool PAD, int D = HD>
__global__ __launch_bounds__(256) void k_probs(ProbsArgs a) {
  extern __shared__ __align__(16) __bf16 lds_dyn[];
  using Ly = ProbsLayout<IO, M, D>;
  constexpr int NS = Ly::NS, KS = Ly::KS, TM = M / 16, DK = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  // blocks i, i + 8, ... (same XCD) take the column blocks of one token block
  const int grp = blockIdx.x / (8 * Ly::NCB), w8 = blockIdx.x % (8 * Ly::NCB);
  const int cb = w8 / 8, tw0 = (grp * 8 + (w8 % 8)) * PROBS_TOK * a.grp;
  if (tw0 >= a.n) return;  // whole workgroup, before any barrier
  int t0 = tw0;
  const int col0 = cb * PROBS_CB;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + a.in.base(bh, a.H);
  const long long st = a.in.t;

  const __bf16* const src_h = a.kt_hi + (size_t)bh * M * D;
  const __bf16* const src_l = a.kt_lo + (size_t)bh * M * D;
  __bf16* const kth_lds = lds_dyn;
  __bf16* const ktl_lds = kth_lds + Ly::KT_ELEMS;
  const __bf16* const kth = Ly::KT_LDS ? kth_lds : src_h;
  const __bf16* const ktl = Ly::KT_LDS ? ktl_lds : src_l;
  constexpr int KROW = Ly::KT_LDS ? Ly::KLD : D;
  __bf16* const zfh = lds_dyn + Ly::OFF_ZF;
  __bf16* const zfl = zfh + Ly::ZF_ELEMS;

  // Q B fragments of both tiles, in flight with the staging
  Frag2 qf2[2][DK];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tok = min(t0 + 32 * wave + 16 * u + c16, a.n - 1);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      float x[8];
      IOTraits<IO>::load8(Q + tok * st + 32 * ks + 8 * g, x);
      qf2[u][ks] = make_frag<NS>(x);
    }
  }
  {
    if constexpr (Ly::KT_LDS) {
      for (int idx = threadIdx.x; idx < M * (D / 8); idx += 256) {
        const int row = idx / (D / 8), cc = idx % (D / 8);
        *reinterpret_cast<bf16x8*>(kth_lds + row * Ly::KLD + 8 * cc) =
            *reinterpret_cast<const bf16x8*>(src_h + (size_t)row * D + 8 * cc);
        if constexpr (NS == 3)
          *reinterpret_cast<bf16x8*>(ktl_lds + row * Ly::KLD + 8 * cc) =
              *reinterpret_cast<const bf16x8*>(src_l + (size_t)row * D + 8 * cc);
      }
    }
    // fragment (jt, ks), lane l: Z^T[col0 + 16 jt + l % 16][k] for the paired
    // k order of the S^T tiles, k = 32 ks + 4 (l / 16) + e (+ 12 for e >= 4)
    const float* Zh = a.Z + (size_t)bh * M * M;
    for (int idx = threadIdx.x; idx < 4 * KS * 64; idx += 256) {
      const int l = idx & 63, f = idx >> 6;
      const int jt = f / KS, ks = f % KS;
      const int gg = l >> 4, col = col0 + 16 * jt + (l & 15);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 32 * ks + 4 * gg + (e < 4 ? e : 12 + e);
        x[e] = col < M ? Zh[(size_t)kk * M + col] : 0.f;
      }
      const Frag2 zf = split8(x);
      *reinterpret_cast<bf16x8*>(zfh + 8 * idx) = zf.hi;
      *reinterpret_cast<bf16x8*>(zfl + 8 * idx) = zf.lo;
    }
  }
  __syncthreads();

  for (int gi = 0; gi < a.grp; ++gi) {
  t0 = tw0 + gi * PROBS_TOK;
  if (t0 >= a.n) break;
  if (gi > 0) {  // this group's Q fragments
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = min(t0 + 32 * wave + 16 * u + c16, a.n - 1);
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        float x[8];
        IOTraits<IO>::load8(Q + tok * st + 32 * ks + 8 * g, x);
        qf2[u][ks] = make_frag<NS>(x);
      }
    }
  }
  const int njt = min(4, (M - col0) / 16);
  const bool vec = (a.ldp & 3) == 0;
  const float ls2 = a.lscale * LOG2E;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;
    if (ts >= a.n) break;
    const int tok = ts + c16;
    const Frag2(&qf)[DK] = qf2[u];
    f32x4 sacc[TM];
#pragma unroll
    for (int it = 0; it < TM; ++it) {
      sacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        Frag2 kf;
        const int off = (16 * it + c16) * KROW + 32 * ks + 8 * g;
        kf.hi = *reinterpret_cast<const bf16x8*>(kth + off);
        if constexpr (NS == 3) kf.lo = *reinterpret_cast<const bf16x8*>(ktl + off);
        sacc[it] = mma<NS>(kf, qf[ks], sacc[it]);
      }
    }
    if constexpr (PAD) pad_mask_rows(sacc, a.mr);
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[it][r]);
    const float mb = max_g(mx) * ls2;
    float sum = 0.f;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(sacc[it][r], ls2, -mb));
        sacc[it][r] = p;
        sum += p;
      }
    const float inv = 1.0f / sum_g(sum);
    f32x4 pacc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) pacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8] = {sacc[2 * ks][0] * inv,     sacc[2 * ks][1] * inv,     sacc[2 * ks][2] * inv,
                    sacc[2 * ks][3] * inv,     sacc[2 * ks + 1][0] * inv, sacc[2 * ks + 1][1] * inv,
                    sacc[2 * ks + 1][2] * inv, sacc[2 * ks + 1][3] * inv};
      const Frag2 pf = split8(x);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt >= njt) break;
        Frag2 zf;
        const int off = ((jt * KS + ks) * 64 + lane) * 8;
        zf.hi = *reinterpret_cast<const bf16x8*>(zfh + off);
        zf.lo = *reinterpret_cast<const bf16x8*>(zfl + off);
        pacc[jt] = mma<3>(zf, pf, pacc[jt]);
      }
    }
    if (tok < a.n) {
      IO* const row = reinterpret_cast<IO*>(a.probs) + ((size_t)bh * a.n + tok) * a.ldp;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt >= njt) break;
        store_probs4<IO>(row, col0 + 16 * jt + 4 * g, a.mr, vec, pacc[jt]);
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Exact branch.  grid: (ceil(n / (4 xprobs_q<D>())), BH), block 256, no LDS.
// Query rows per wave: 4 tiles of 16 (2 at d = 128, for registers).
template <int D>
constexpr int xprobs_q() {
  return D > 64 ? 32 : 64;
}

template <typename IO, int D>
__device__ __forceinline__ void xprobs_key_frags(const IO* K, long long st, int n, int key0, Frag2 (&kf)[D / 32]) {
  constexpr int NS = IOTraits<IO>::NS;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int key = min(key0 + c16, n - 1);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    float x[8];
    IOTraits<IO>::load8(K + key * st + 32 * ks + 8 * g, x);
    kf[ks] = make_frag<NS>(x);
  }
}

// logits of keys key0 + 4g + r (rows of the S^T tile) for query tile o,
// in log2 units; -inf for keys past n or masked
template <int NS, int DK>
__device__ __forceinline__ f32x4 xprobs_logits(const Frag2 (&kf)[DK], const Frag2 (&qf)[DK], const bool (&valid)[4],
                                               float ls2) {
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) s = mma<NS>(kf[ks], qf[ks], s);
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = valid[r] ? s[r] * ls2 : -INFINITY;
  return s;
}

template <typename IO, int D = HD>
__global__ __launch_bounds__(256) void k_exact_probs(ProbsArgs a) {
  constexpr int NS = IOTraits<IO>::NS, DK = D / 32, QT = xprobs_q<D>() / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H;
  const int q0 = blockIdx.x * 4 * xprobs_q<D>() + xprobs_q<D>() * wave;
  if (q0 >= a.n) return;  // whole wave; the kernel has no barriers
  const int nown = min(QT, (a.n - q0 + 15) / 16);
  const IO* Q = reinterpret_cast<const IO*>(a.q) + a.in.base(bh, a.H);
  const IO* K = reinterpret_cast<const IO*>(a.k) + a.in.base(bh, a.H);
  const long long st = a.in.t;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  const float ls2 = a.lscale * LOG2E;

  Frag2 qf[QT][DK];
#pragma unroll
  for (int o = 0; o < QT; ++o) {
    const int tok = min(q0 + 16 * o + c16, a.n - 1);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      float x[8];
      IOTraits<IO>::load8(Q + tok * st + 32 * ks + 8 * g, x);
      qf[o][ks] = make_frag<NS>(x);
    }
  }
  auto key_valid = [&](int key0, bool(&valid)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * g + r;
      bool v = key < a.n;
      if (mask != nullptr && v) v = mask[key] != 0;
      valid[r] = v;
    }
  };

  // pass 1: per lane, running maximum and sum over its keys of every tile
  float mrun[QT], lsum[QT];
#pragma unroll
  for (int o = 0; o < QT; ++o) {
    mrun[o] = NEG_BIG;
    lsum[o] = 0.f;
  }
  for (int key0 = 0; key0 < a.n; key0 += 16) {
    Frag2 kf[DK];
    xprobs_key_frags<IO, D>(K, st, a.n, key0, kf);
    bool valid[4];
    key_valid(key0, valid);
#pragma unroll
    for (int o = 0; o < QT; ++o) {
      if (o >= nown) break;
      const f32x4 s = xprobs_logits<NS, DK>(kf, qf[o], valid, ls2);
      const float mnew = fmaxf(mrun[o], fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
      lsum[o] = lsum[o] * fast_exp2(mrun[o] - mnew) + fast_exp2(s[0] - mnew) + fast_exp2(s[1] - mnew) +
                fast_exp2(s[2] - mnew) + fast_exp2(s[3] - mnew);
      mrun[o] = mnew;
    }
  }
  float inv[QT];
#pragma unroll
  for (int o = 0; o < QT; ++o) {
    const float mrow = max_g(mrun[o]);
    const float srow = sum_g(lsum[o] * fast_exp2(mrun[o] - mrow));
    mrun[o] = mrow;
    inv[o] = srow > 0.f ? 1.0f / srow : 0.f;
  }

  // pass 2: normalised weights
  const bool vec = (a.n & 3) == 0;
  for (int key0 = 0; key0 < a.n; key0 += 16) {
    Frag2 kf[DK];
    xprobs_key_frags<IO, D>(K, st, a.n, key0, kf);
    bool valid[4];
    key_valid(key0, valid);
#pragma unroll
    for (int o = 0; o < QT; ++o) {
      if (o >= nown) break;
      const f32x4 s = xprobs_logits<NS, DK>(kf, qf[o], valid, ls2);
      f32x4 p;
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] - mrun[o]) * inv[o];
      const int tok = q0 + 16 * o + c16;
      if (tok < a.n)
        store_probs4<IO>(reinterpret_cast<IO*>(a.probs) + ((size_t)bh * a.n + tok) * a.ldp, key0 + 4 * g, a.n, vec,
                         p);
    }
  }
}

}  // namespace nys
