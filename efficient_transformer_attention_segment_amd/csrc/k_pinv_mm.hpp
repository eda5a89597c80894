// Iterative Moore-Penrose inverse for more than 128 landmarks (bf16 I/O):
// a launch sequence over global memory, three launches per iteration.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.5:
// Z_0 = A^T / c, then n_iter times X = A Z and
// Z <- (1/4) Z (13 I - X (15 I - X (7 I - X))).
//
// The update is evaluated with the product expanded,
//   Z' = (13 Z - 15 Z X + 7 Z X^2 - Z X^3) / 4,
// which equals the nested form in exact arithmetic, as
//   level 1  X  = A Z
//   level 2  X2 = X X  and  W = Z X          (independent: one launch)
//   level 3  Z' = (13 Z - 15 W + 7 W X - W X2) / 4
// X is still recomputed from A and Z every iteration (self-correcting).
// Every product operand is a matrix the iteration produced (Z, X, W, X2),
// never a shifted difference such as 13 I - T2 whose rounding to a 16-bit
// operand loses its small part: with single fp16 products this order keeps
// the iterate within about 1e-4 of the float64 iteration where the nested
// order, rounded the same way, drifts by several per cent.  The linear
// combinations run in float32 in the epilogues.
//
// gram_rows_body: A = softmax(Qt Kt^T) by 32-row blocks, split-bf16
//   products as in the one-block Gram; writes A, A^T and per row block the
//   column sums and the largest row sum.  At d = 64 it runs in the first
//   workgroups of the B V launch, otherwise as k_gram_rows.
// k_pinv_mm<LEVEL>: 32 x 32 output tiles (4 waves of one 16 x 16 tile
//   each, K = M in fp16 16x16x32 matrix-core steps), every tile of a head on
//   one XCD.  Level 1 of the first iteration also forms c from the Gram
//   partials (column sums of the row blocks added in order).  Operand
//   panels are 32 rows of the left factor and 32 rows of the right factor's
//   transpose, copied into LDS once per block.  The matrices that serve as
//   operands are kept in global memory as fp16 rows (A, X, X^T, (X^2)^T, W,
//   Z, Z^T), rounded once by the launch that forms them: each workgroup's
//   inputs come from the Infinity Cache at a rate of a few tens of GB/s per
//   CU, so halving the bytes of its two or three panels is what shortens the
//   launch.  Z and W are also kept in float32 for the linear combination.
//   In the first iteration Z = A^T / c is read from the float32 A^T (rows of
//   Z) and A (rows of Z^T), scaled and rounded on the way into LDS.
#pragma once

#include "common.hpp"
#include "k_landmark.hpp"
#include "k_pinv.hpp"

namespace nys {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ Gram rows ---
// A = softmax(Qt Kt^T) by 32-row blocks, for the B V launch: its first
// gram_rows_blocks() workgroups run this instead of B V partials (the
// launch's blocks have four waves; a wave pair forms one 32-row block, so a
// workgroup covers two row blocks of one head), which saves a launch of its
// own before the B V stream.
template <int M, int D>
constexpr int gram_rows_lds_bytes() {
  return 2 * M * (D + 8) * 2 + 4 * (4 * M + 4);
}
// row-block pairs per head
template <int M>
constexpr int gram_rows_per_head() {
  return (M / 32 + 1) / 2;
}
template <int M>
inline int gram_rows_blocks(int BH) {
  return BH * gram_rows_per_head<M>();
}

// Workgroup blk (256 threads): head blk / gram_rows_per_head, wave w forms
// row tile 2 rb + (w & 1) of row block rb = 2 (blk % gram_rows_per_head) +
// (w >> 1) (a wave pair past the last row block only meets the barriers).
// Writes A (float32 and fp16), A^T (float32) and, per row block, the column
// sums and the largest row sum.
template <int M, int D>
__device__ void gram_rows_body(const LandmarkArgs& a, float* __restrict__ AT, u16* __restrict__ A16,
                               float* __restrict__ colpart, float* __restrict__ rowpart, int blk, char* gr_smem) {
  constexpr int TM = M / 16, DK = D / 32, KLD = D + 8, NT = 256, RB = M / 32;
  __bf16* const kb = reinterpret_cast<__bf16*>(gr_smem);  // hi rows 0 .. M-1, lo rows M .. 2M-1
  float* const csum = reinterpret_cast<float*>(gr_smem + 2 * M * KLD * 2);  // [4 waves][M]
  float* const rmx = csum + 4 * M;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blk / gram_rows_per_head<M>();
  const int rb = 2 * (blk % gram_rows_per_head<M>()) + (wave >> 1);
  const bool live = rb < RB;
  const int rt = 2 * rb + (wave & 1);
  {
    // the K~ planes into LDS in batches of 4 pieces per thread, every load of
    // a batch issued before its stores (one round trip per batch instead of
    // one per piece)
    const uint4* kh = reinterpret_cast<const uint4*>(a.kt_hi + (size_t)bh * M * D);
    const uint4* kl = reinterpret_cast<const uint4*>(a.kt_lo + (size_t)bh * M * D);
    constexpr int PIECES = M * (D / 8), PER = (PIECES + NT - 1) / NT, BATCH = 4;
#pragma unroll
    for (int b0 = 0; b0 < PER; b0 += BATCH) {
      uint4 xh[BATCH], xl[BATCH];
      // every element is assigned (an index past the planes reads piece 0
      // and is not stored), so the arrays stay in registers
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = threadIdx.x + NT * (b0 + j);
        const int ic = (b0 + j < PER && i < PIECES) ? i : 0;
        xh[j] = kh[ic];
        xl[j] = kl[ic];
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = threadIdx.x + NT * (b0 + j);
        if (b0 + j < PER && i < PIECES) {
          *reinterpret_cast<uint4*>(kb + (i / (D / 8)) * KLD + 8 * (i % (D / 8))) = xh[j];
          *reinterpret_cast<uint4*>(kb + (M + i / (D / 8)) * KLD + 8 * (i % (D / 8))) = xl[j];
        }
      }
    }
  }
  Frag2 af[DK];
  if (live) {
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const size_t off = ((size_t)bh * M + rt * 16 + c16) * D + ks * 32 + g * 8;
      af[ks].hi = *reinterpret_cast<const bf16x8*>(a.qt_hi + off);
      af[ks].lo = *reinterpret_cast<const bf16x8*>(a.qt_lo + off);
    }
  }
  __syncthreads();
  float rmax_w = 0.f;
  if (live) {
    f32x4 acc[TM];
#pragma unroll
    for (int ct = 0; ct < TM; ++ct) {
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const int row = ct * 16 + c16, col = ks * 32 + g * 8;
        Frag2 bf;
        bf.hi = *reinterpret_cast<const bf16x8*>(kb + row * KLD + col);
        bf.lo = *reinterpret_cast<const bf16x8*>(kb + (M + row) * KLD + col);
        acc[ct] = mma<3>(af[ks], bf, acc[ct]);
      }
    }
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
      rmax_w = fmaxf(rmax_w, sum16(rs));
    }
    float* const Ah = a.A + (size_t)bh * M * M;
    float* const ATh = AT + (size_t)bh * M * M;
    _Float16* const A16h = reinterpret_cast<_Float16*>(A16) + (size_t)bh * M * M;
    const int row4 = rt * 16 + 4 * g;
#pragma unroll
    for (int ct = 0; ct < TM; ++ct) {
      const int col = ct * 16 + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Ah[(size_t)(row4 + r) * M + col] = acc[ct][r];
        A16h[(size_t)(row4 + r) * M + col] = (_Float16)acc[ct][r];
      }
      *reinterpret_cast<float4*>(ATh + (size_t)col * M + row4) =
          make_float4(acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
      const float cs = sum_g(acc[ct][0] + acc[ct][1] + acc[ct][2] + acc[ct][3]);
      if (g == 0) csum[wave * M + col] = cs;
    }
  }
  rmax_w = max_g(rmax_w);
  if (lane == 0) rmx[wave] = rmax_w;
  __syncthreads();
  // the row block of each wave pair: column sums of its two row tiles
  // (added in the order of the tiles) and its largest row sum
  const int pr = threadIdx.x >> 7, pt = threadIdx.x & 127;  // pair, thread within the pair
  const int rbp = 2 * (blk % gram_rows_per_head<M>()) + pr;
  if (rbp < RB) {
    float* const cp = colpart + ((size_t)bh * RB + rbp) * M;
    for (int j = pt; j < M; j += 128) cp[j] = csum[(2 * pr) * M + j] + csum[(2 * pr + 1) * M + j];
    if (pt == 0) rowpart[(size_t)bh * RB + rbp] = fmaxf(rmx[2 * pr], rmx[2 * pr + 1]);
  }
}

// The same as a launch of its own (head sizes other than 64, whose B V
// launch keeps its own LDS plan): grid gram_rows_blocks(BH), 256 threads.
template <int M, int D>
__global__ __launch_bounds__(256) void k_gram_rows(LandmarkArgs a, float* __restrict__ AT, u16* __restrict__ A16,
                                                   float* __restrict__ colpart, float* __restrict__ rowpart) {
  extern __shared__ __align__(16) char gr_smem[];
  gram_rows_body<M, D>(a, AT, A16, colpart, rowpart, blockIdx.x, gr_smem);
}

// -------------------------------------------------------------- products ---
struct PinvMMArgs {
  // [BH][M][M] each; fp16 matrices as _Float16 bit patterns
  const float* A;    // rows of A (float32: the first iteration's Z^T = A / c)
  const float* AT;   // rows of A^T (float32: the first iteration's Z = A^T / c)
  const u16* A16;    // rows of A
  float* Z;          // rows of Z (float32), updated in place by level 3
  u16* Z16;          // rows of Z
  u16* Zt16;         // rows of Z^T
  u16* X16;          // rows of X
  u16* Xt16;         // rows of X^T
  u16* X2t16;        // rows of (X^2)^T
  float* W;          // rows of W = Z X (float32)
  u16* W16;          // rows of W
  const float* colpart;  // [BH][M / 32][M] Gram column-sum partials
  const float* rowpart;  // [BH][M / 32] Gram row-sum maxima
  float* colmax;     // [BH] out: head's largest column sum of A
  float* rowmax;     // [BH] out: head's largest row sum of A
  PinvArgs pa;       // BH, init option; cscale out
  int first;         // 1: k = 0, Z = A^T / c
};

constexpr int PMM_T = 32;  // output tile

template <int M>
constexpr int pinv_mm_ld() {
  return M + 8;  // fp16 panel row stride (16-byte chunks land on distinct banks)
}
template <int M, int LEVEL>
constexpr int pinv_mm_lds_bytes() {
  return (LEVEL == 3 ? 3 : 2) * PMM_T * pinv_mm_ld<M>() * 2;
}

// Rows r0 .. r0 + 31 of a float32 [M][M] matrix, times s, as fp16 rows of
// an LDS panel (row stride pinv_mm_ld): the loads first (N float4 per
// thread), then the stores.
template <int M>
struct PanelLoad {
  static constexpr int N = PMM_T * M / 4 / 256;
  float4 x[N];
  __device__ __forceinline__ void load(const float* src, int r0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + 256 * i;  // float4 index within the panel
      x[i] = *reinterpret_cast<const float4*>(src + (size_t)(r0 + idx / (M / 4)) * M + 4 * (idx % (M / 4)));
    }
  }
  __device__ __forceinline__ void store(_Float16* lds, float s) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + 256 * i;
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 h = {(_Float16)(x[i].x * s), (_Float16)(x[i].y * s), (_Float16)(x[i].z * s), (_Float16)(x[i].w * s)};
      *reinterpret_cast<h4*>(lds + (idx / (M / 4)) * pinv_mm_ld<M>() + 4 * (idx % (M / 4))) = h;
    }
  }
};

// Rows r0 .. r0 + 31 of an fp16 [M][M] matrix into an LDS panel: the loads
// first (N 16-byte pieces per thread), then the stores.
template <int M>
struct PanelLoad16 {
  static constexpr int TOT = PMM_T * M / 8, N = (TOT + 255) / 256;  // 8-element pieces
  uint4 x[N];
  __device__ __forceinline__ void load(const u16* src, int r0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int idx = threadIdx.x + 256 * i;  // piece index within the panel
      if (TOT % 256 != 0 && idx >= TOT) idx = 0;  // past the panel: a valid address, not stored
      x[i] = *reinterpret_cast<const uint4*>(src + (size_t)(r0 + idx / (M / 8)) * M + 8 * (idx % (M / 8)));
    }
  }
  __device__ __forceinline__ void store(_Float16* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (TOT % 256 == 0 || idx < TOT)
        *reinterpret_cast<uint4*>(lds + (idx / (M / 8)) * pinv_mm_ld<M>() + 8 * (idx % (M / 8))) = x[i];
    }
  }
};

// Panel from float32 rows times s (first iteration) or from fp16 rows.
template <int M>
__device__ __forceinline__ void load_panel(_Float16* lds, bool f32, const float* src32, float s, const u16* src16,
                                           int r0) {
  if (f32) {
    PanelLoad<M> l;
    l.load(src32, r0);
    l.store(lds, s);
  } else {
    PanelLoad16<M> l;
    l.load(src16, r0);
    l.store(lds);
  }
}

// C tile (16 x 16) of the wave: sum_k Lp[16 it + i][k] Rp[16 jt + j][k].
template <int M>
__device__ __forceinline__ f32x4 panel_mm(const _Float16* Lp, const _Float16* Rp, int it, int jt) {
  constexpr int LD = pinv_mm_ld<M>();
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const _Float16* pa = Lp + (16 * it + c16) * LD + 8 * g;
  const _Float16* pb = Rp + (16 * jt + c16) * LD + 8 * g;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    const h16x8 av = *reinterpret_cast<const h16x8*>(pa + 32 * ks);
    const h16x8 bv = *reinterpret_cast<const h16x8*>(pb + 32 * ks);
    acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[ks & 1], 0, 0, 0);
  }
  return acc[0] + acc[1];
}

// Stores the wave's C tile (rows row4 .. row4 + 3, column col) of a
// product: float32 rows into C32, fp16 rows into C16 and fp16 rows of the
// transpose into Ct16, each when given.
__device__ __forceinline__ void store_c(float* C32, u16* C16, u16* Ct16, int M, int row4, int col, const f32x4 v) {
  if (C32 != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) C32[(size_t)(row4 + r) * M + col] = v[r];
  }
  if (C16 != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) reinterpret_cast<_Float16*>(C16)[(size_t)(row4 + r) * M + col] = (_Float16)v[r];
  }
  if (Ct16 != nullptr) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<h4*>(Ct16 + (size_t)col * M + row4) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  }
}

// Workgroups per launch: tiles per head (T = (M / 32)^2 for levels 1 and
// 3, 2 T for level 2: X2 tiles, then W tiles) for every head, placed so that
// all of a head's tiles run on one XCD (workgroup i of a launch runs on XCD
// i mod 8): the matrices one launch writes are then read by the next from
// the L2 of the XCD that wrote them.  Heads h and h + 8 share XCD h mod 8.
__host__ __device__ constexpr int pinv_mm_grid(int tiles, int BH) { return 8 * tiles * ((BH + 7) / 8); }

// c for head bh from the Gram partials (gram_rows_body): the largest column sum
// (row blocks added in order) times the largest row sum, over every head for
// the original init, over head bh alone for the exact-coefficient init.  Also
// head bh's own two maxima.  Whole workgroup (256 threads); red: 12 floats.
template <int M>
__device__ float pinv_c_from_parts(const float* colpart, const float* rowpart, int bh, int BH, int init_option,
                                   float* red, float& cm_own, float& rm_own) {
  constexpr int NB = M / 32;
  const int h0 = init_option == 0 ? 0 : bh, h1 = init_option == 0 ? BH : bh + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float cm = 0.f, rm = 0.f, cmo = 0.f, rmo = 0.f;
  for (int i = threadIdx.x; i < (h1 - h0) * M; i += 256) {
    const int h = h0 + i / M, j = i % M;
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) s += colpart[((size_t)h * NB + b) * M + j];
    cm = fmaxf(cm, s);
    if (h == bh) cmo = fmaxf(cmo, s);
  }
  for (int i = threadIdx.x; i < (h1 - h0) * NB; i += 256) {
    const float r = rowpart[(size_t)h0 * NB + i];
    rm = fmaxf(rm, r);
    if (h0 + i / NB == bh) rmo = fmaxf(rmo, r);
  }
  cm = wave_max(cm);
  rm = wave_max(rm);
  cmo = wave_max(cmo);
  rmo = wave_max(rmo);
  if (lane == 0) {
    red[wave] = cm;
    red[4 + wave] = rm;
    red[8 + wave] = cmo;
    red[12 + wave] = rmo;
  }
  __syncthreads();
  auto max4 = [&](int o) { return fmaxf(fmaxf(red[o], red[o + 1]), fmaxf(red[o + 2], red[o + 3])); };
  cm_own = max4(8);
  rm_own = max4(12);
  return max4(0) * max4(4);
}

template <int M, int LEVEL>
__global__ __launch_bounds__(256) void k_pinv_mm(PinvMMArgs a) {
  extern __shared__ __align__(16) _Float16 pm_lds[];
  __shared__ float red[16];
  constexpr int NT = M / PMM_T, LD = pinv_mm_ld<M>(), PANEL = PMM_T * LD;
  constexpr int TILES = (LEVEL == 2 ? 2 : 1) * NT * NT;
  const int L = blockIdx.x, xcd = L & 7, s = L >> 3;
  // Every tile of a head on one XCD (its operand panels then come into one
  // L2); with at most four heads a head takes two XCDs, x and x + 4, each
  // half of its tiles, so each CU holds one workgroup instead of two
  // (what bounds a launch is the rate at which a CU receives its panels).
  int bh, t2;
  if (a.pa.BH <= 4) {
    constexpr int H0 = (TILES + 1) / 2;
    bh = xcd & 3;
    t2 = (xcd >> 2) * H0 + s;
    if (s >= H0 || t2 >= TILES) return;  // whole workgroup, before any barrier
  } else {
    bh = xcd + 8 * (s / TILES);
    t2 = s % TILES;
  }
  if (bh >= a.pa.BH) return;  // whole workgroup, before any barrier
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const bool second = LEVEL == 2 && t2 >= NT * NT;  // level 2: the W = Z X tiles
  const int tile = second ? t2 - NT * NT : t2;
  const int ti = tile / NT, tj = tile % NT;
  const size_t mo = (size_t)bh * M * M;
  // 1 / c: level 1 of the first iteration forms c from the Gram partials
  // (and writes it with the head's maxima); later launches read it back
  float invc = 1.f;
  if (a.first) {
    if (LEVEL == 1) {
      float cmo, rmo;
      const float c = pinv_c_from_parts<M>(a.colpart, a.rowpart, bh, a.pa.BH, a.pa.init_option, red, cmo, rmo);
      if (tile == 0 && threadIdx.x == 0) {
        a.pa.cscale[bh] = c;
        a.colmax[bh] = cmo;
        a.rowmax[bh] = rmo;
      }
      invc = 1.0f / c;
    } else {
      invc = 1.0f / a.pa.cscale[bh];
    }
  }
  // float32 rows of Z (A^T / c in the first iteration) for level 3
  const float* const Zr = a.first ? a.AT + mo : a.Z + mo;
  _Float16* const P0 = pm_lds;
  _Float16* const P1 = pm_lds + PANEL;
  _Float16* const P2 = pm_lds + 2 * PANEL;
  const int r0 = PMM_T * ti, c0 = PMM_T * tj;
  if constexpr (LEVEL == 1) {  // X = A Z: rows of A, rows of Z^T (A / c first)
    PanelLoad16<M> l;
    l.load(a.A16 + mo, r0);
    load_panel<M>(P1, a.first, a.A + mo, invc, a.Zt16 + mo, c0);
    l.store(P0);
  } else if constexpr (LEVEL == 2) {  // X2 = X X, or W = Z X (Z = A^T / c first)
    PanelLoad16<M> r;
    r.load(a.Xt16 + mo, c0);
    if (second)
      load_panel<M>(P0, a.first, a.AT + mo, invc, a.Z16 + mo, r0);
    else
      load_panel<M>(P0, false, nullptr, 1.f, a.X16 + mo, r0);
    r.store(P1);
  } else {  // Z' = (13 Z - 15 W + 7 W X - W X2) / 4
    PanelLoad16<M> l, r1, r2;
    l.load(a.W16 + mo, r0);
    r1.load(a.Xt16 + mo, c0);
    r2.load(a.X2t16 + mo, c0);
    l.store(P0);
    r1.store(P1);
    r2.store(P2);
  }
  __syncthreads();
  const int it = wave >> 1, jt = wave & 1;
  const int row4 = r0 + 16 * it + 4 * g, col = c0 + 16 * jt + c16;
  const f32x4 acc = panel_mm<M>(P0, P1, it, jt);
  if constexpr (LEVEL == 1) {
    store_c(nullptr, a.X16 + mo, a.Xt16 + mo, M, row4, col, acc);
  } else if constexpr (LEVEL == 2) {
    if (second)
      store_c(a.W + mo, a.W16 + mo, nullptr, M, row4, col, acc);
    else  // X^2 is only ever a right factor: its transpose alone
      store_c(nullptr, nullptr, a.X2t16 + mo, M, row4, col, acc);
  } else {
    const f32x4 v = panel_mm<M>(P0, P2, it, jt);
    f32x4 z;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float zr = Zr[(size_t)(row4 + r) * M + col] * invc;
      const float wr = a.W[mo + (size_t)(row4 + r) * M + col];
      z[r] = 0.25f * (13.f * zr - 15.f * wr + 7.f * acc[r] - v[r]);
    }
    // over Z in place: this tile is the only reader of its float32 Z
    store_c(a.Z + mo, a.Z16 + mo, a.Zt16 + mo, M, row4, col, z);
  }
}

}  // namespace nys
