// Streamed softmax-weighted sums over the keys: B V for the Nystrom path
// and the exact-attention branch.
//
// Pages: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4
// (kernel_3 B = softmax(Qt Ks^T + mask), the only place the mask enters, and
// new_value = B V) and section 2.1 (exact attention when m equals n);
// Hugging Face Transformers docs (zh), Nystromformer model page
// (attention_mask: 1 keeps a token, 0 masks it).
//
// A workgroup owns up to 64 "columns" (landmarks for B V, queries for the
// exact branch; 16 per wave and tile) and streams 32-key tiles of K and V
// through LDS.  bf16 inputs are copied global -> LDS by DMA, six tiles
// ahead (K and V row-major; V read back transposed by ds_read_b64_tr_b16);
// float32 inputs go through registers (split into bf16 hi/lo, V stored
// transposed), double buffered.  Per tile and wave:
//   S^T (32 keys x 16 columns) = K_tile Qcol^T on the matrix cores,
//   an online softmax down each column (running max / sum, the row max taken
//   over the four lane groups by cross-lane shuffles),
//   acc^T (64 d x 16 columns) += V_tile^T P^T, with the probabilities used
//   straight from the S^T C tile as the B operand (paired k order).
// The m x n matrix B never leaves registers.  Masked keys get weight 0; a
// column that saw no valid key keeps max = -1e30, sum = 0, acc = 0.  Partial
// maxima are written in log2 units of the scaled logit.
#pragma once

#include "common.hpp"
#include "k_conv.hpp"
#include "k_pinv.hpp"
#include "k_pinv_mm.hpp"

namespace nys {

template <typename IO, int D = HD>
struct KV {
  static constexpr int NS = IOTraits<IO>::NS;
  static constexpr int KT = 32;         // keys per tile
  static constexpr int KLD = D + 8;     // K tile row stride (bf16 elements)
  static constexpr int VLD = KT + 8;    // V^T tile row stride
  static constexpr int K_ELEMS = KT * KLD;
  static constexpr int V_ELEMS = D * VLD;
  static constexpr int PART = K_ELEMS + V_ELEMS;                 // hi (or lo) part
  static constexpr int BUF_ELEMS = PART * (NS == 3 ? 2 : 1);
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;            // two buffers
};

// Register staging: the 32 x (D / 8) (row, 8-channel chunk) items of a
// 32-key tile are spread over the NT threads of the block (N per thread).
template <int NT, int D = HD>
struct Items {
  static constexpr int ALL = 4 * D;
  static constexpr int N = (ALL + NT - 1) / NT;
};

template <typename IO, int NT, int D = HD>
__device__ __forceinline__ void kv_load(const IO* __restrict__ K, const IO* __restrict__ V, long long st, int n,
                                        int key0, float (&kx)[Items<NT, D>::N][8], float (&vx)[Items<NT, D>::N][8]) {
#pragma unroll
  for (int u = 0; u < Items<NT, D>::N; ++u) {
    const int item = threadIdx.x + u * NT;
    const int row = key0 + item / (D / 8), cc = item % (D / 8);
    if (item < Items<NT, D>::ALL && row < n) {
      IOTraits<IO>::load8(K + row * st + 8 * cc, kx[u]);
      IOTraits<IO>::load8(V + row * st + 8 * cc, vx[u]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[u][e] = vx[u][e] = 0.f;
    }
  }
}

template <typename IO, int NT, int D = HD>
__device__ __forceinline__ void kv_store(__bf16* buf, const float (&kx)[Items<NT, D>::N][8],
                                         const float (&vx)[Items<NT, D>::N][8]) {
  using C = KV<IO, D>;
#pragma unroll
  for (int u = 0; u < Items<NT, D>::N; ++u) {
    const int item = threadIdx.x + u * NT;
    if (item >= Items<NT, D>::ALL) continue;
    const int kk = item / (D / 8), cc = item % (D / 8);
    const Frag2 kf = make_frag<C::NS>(kx[u]);
    *reinterpret_cast<bf16x8*>(buf + kk * C::KLD + 8 * cc) = kf.hi;
    if constexpr (C::NS == 3) *reinterpret_cast<bf16x8*>(buf + C::PART + kk * C::KLD + 8 * cc) = kf.lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split1(vx[u][e], h, l);
      buf[C::K_ELEMS + (8 * cc + e) * C::VLD + kk] = h;
      if constexpr (C::NS == 3) buf[C::PART + C::K_ELEMS + (8 * cc + e) * C::VLD + kk] = l;
    }
  }
}

// Per-tile math shared by both staging paths: S^T from the K fragments,
// masked online softmax per column, acc^T += V^T P^T.
//
// The running column maximum mrun is kept in log2 units of the scaled logit
// (x = s * lscale * log2 e).  Probabilities are taken against the stored
// maximum, p = 2^(x - mrun), which is exact after the final division by the
// running sum; the maximum (a cross-lane reduction over the four lane
// groups) and the rescale of sum and accumulators are only redone when some
// logit in the wave exceeds its stored maximum by RESCALE_LOG2 (p stays
// below 2^8, far from float overflow).  A wave-uniform vote picks the path.
constexpr float RESCALE_LOG2 = 8.f;

template <int NS, int TPW, bool MASKED, int D = HD>
__device__ __forceinline__ void kv_compute(const Frag2 (&kf)[2][D / 32], const Frag2 (&vf)[D / 16],
                                           const bool (&valid)[8], const Frag2 (&qf)[TPW][D / 32], int nown,
                                           float lscale2, float (&mrun)[TPW], float (&lsum)[TPW],
                                           f32x4 (&acc)[TPW][D / 16]) {
#pragma unroll
  for (int o = 0; o < TPW; ++o) {
    if (o >= nown) break;
    f32x4 s[2];
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      s[kst] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) s[kst] = mma<NS>(kf[kst][ks], qf[o][ks], s[kst]);
    }
    // raw logits (the scale is positive, so the maximum is taken before it
    // and the scale enters the exponent's fma: one VALU op less per key)
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[kst][r];
        if constexpr (MASKED) v = valid[4 * kst + r] ? v : -INFINITY;
        x[4 * kst + r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax *= lscale2;
    if (__builtin_amdgcn_ballot_w64(tmax > mrun[o] + RESCALE_LOG2) != 0) {
      const float mnew = fmaxf(mrun[o], max_g(tmax));
      const float alpha = fast_exp2(mrun[o] - mnew);
      mrun[o] = mnew;
      lsum[o] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[o][dt] *= alpha;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(x[e], lscale2, -mrun[o]));  // a masked key: exp2(-inf) = 0
      lsum[o] += p[e];
    }
    const Frag2 pf = make_frag<NS>(p);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[o][dt] = mma<NS>(vf[dt], pf, acc[o][dt]);
  }
}

// One 32-key tile from the register-staged layout (K row-major, V^T).
template <typename IO, int TPW, int D = HD>
__device__ __forceinline__ void kv_tile_update(const __bf16* buf, const Frag2 (&qf)[TPW][D / 32], int nown, int key0,
                                               int n, const uint8_t* __restrict__ mask, float lscale,
                                               float (&mrun)[TPW], float (&lsum)[TPW], f32x4 (&acc)[TPW][D / 16]) {
  using C = KV<IO, D>;
  constexpr int NS = C::NS;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  bool valid[8];
#pragma unroll
  for (int kst = 0; kst < 2; ++kst)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 * kst + 4 * g + r;
      bool v = key < n;
      if (mask != nullptr && v) v = mask[key] != 0;
      valid[4 * kst + r] = v;
    }
  Frag2 kf[2][D / 32];
#pragma unroll
  for (int kst = 0; kst < 2; ++kst)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int off = (16 * kst + c16) * C::KLD + 32 * ks + 8 * g;
      kf[kst][ks].hi = *reinterpret_cast<const bf16x8*>(buf + off);
      if constexpr (NS == 3) kf[kst][ks].lo = *reinterpret_cast<const bf16x8*>(buf + C::PART + off);
    }
  Frag2 vf[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int off = C::K_ELEMS + dmap<false>(dt, c16) * C::VLD + 4 * g;
    vf[dt].hi = cat44(*reinterpret_cast<const bf16x4*>(buf + off), *reinterpret_cast<const bf16x4*>(buf + off + 16));
    if constexpr (NS == 3)
      vf[dt].lo = cat44(*reinterpret_cast<const bf16x4*>(buf + C::PART + off),
                        *reinterpret_cast<const bf16x4*>(buf + C::PART + off + 16));
  }
  kv_compute<NS, TPW, true, D>(kf, vf, valid, qf, nown, lscale * LOG2E, mrun, lsum, acc);
}

// Stream key tiles [tile0, tile1) of one head through the register-staged
// double buffer (used for float32 I/O and for ragged key ranges).
template <typename IO, int TPW, int NT, int KP = 1, int D = HD>
__device__ __forceinline__ void kv_stream(const IO* __restrict__ K, const IO* __restrict__ V, long long st, int n,
                                          const uint8_t* __restrict__ mask, int tile0, int tile1, float lscale,
                                          __bf16* lds, const Frag2 (&qf)[TPW][D / 32], int nown, float (&mrun)[TPW],
                                          float (&lsum)[TPW], f32x4 (&acc)[TPW][D / 16], int kp = 0) {
  using C = KV<IO, D>;
  float kx[Items<NT, D>::N][8], vx[Items<NT, D>::N][8];
  if (tile0 < tile1) {
    kv_load<IO, NT, D>(K, V, st, n, tile0 * C::KT, kx, vx);
    kv_store<IO, NT, D>(lds, kx, vx);
  }
  __syncthreads();
  for (int tile = tile0; tile < tile1; ++tile) {
    const int cur = (tile - tile0) & 1;
    const bool more = tile + 1 < tile1;
    if (more) kv_load<IO, NT, D>(K, V, st, n, (tile + 1) * C::KT, kx, vx);
    if (((tile - tile0) % KP) == kp)
      kv_tile_update<IO, TPW, D>(lds + cur * C::BUF_ELEMS, qf, nown, tile * C::KT, n, mask, lscale, mrun, lsum,
                                 acc);
    if (more) kv_store<IO, NT, D>(lds + (cur ^ 1) * C::BUF_ELEMS, kx, vx);
    __syncthreads();
  }
}

// ---- bf16 path: K / V tiles copied global -> LDS by DMA ------------------
// Ring of DMA_NBUF tiles of 32 keys (K and V row-major with swizzled
// chunks, plus the tile's 32 mask bytes), DMA_DIST tiles in flight.  Each
// wave issues the copies of 8 K rows, 8 V rows (and the mask tile) per tile.
constexpr int DMA_NBUF = 8, DMA_DIST = 6;
constexpr int DMA_TILE = 32 * HD;  // bf16 elements per K (or V) tile
constexpr int DMA_LDS_BYTES = DMA_NBUF * (2 * DMA_TILE * 2 + 32);

// The 8 wave-wide copies of a tile (4 for the 32 K rows, 4 for the V rows)
// are dealt round-robin to the NW waves; every wave also copies the tile's
// 32 mask bytes (identical data), so each wave issues the same count.
template <int NW, bool MASK>
__device__ __forceinline__ void dma_issue_tile(const u16* __restrict__ K, const u16* __restrict__ V, long long st,
                                               const uint8_t* __restrict__ mask, int key0, __bf16* lds, int buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int id = wave; id < 8; id += NW) {
    const int row = 8 * (id & 3) + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const long long src = (key0 + row) * st + 8 * chunk;
    __bf16* dst = lds + ((id < 4 ? 0 : DMA_NBUF) + buf) * DMA_TILE + 8 * (id & 3) * HD;
    if (id < 4)
      dma16_nt(K + src, dst);  // no later kernel of the forward pass reads K
    else
      dma16(V + src, dst);  // V is read again by the output pass
  }
  if constexpr (MASK) {
    uint8_t* mb = reinterpret_cast<uint8_t*>(lds + 2 * DMA_NBUF * DMA_TILE) + 32 * buf;
    if (lane < 2) dma16(mask + key0 + 16 * lane, mb);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_rt(int k) {
  // wait until at most k * N copies of this wave are outstanding
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<N>(); break;
    case 2: wait_vmcnt<2 * N>(); break;
    case 3: wait_vmcnt<3 * N>(); break;
    case 4: wait_vmcnt<4 * N>(); break;
    default: wait_vmcnt<5 * N>(); break;
  }
}

template <int TPW, bool MASK>
__device__ __forceinline__ void dma_tile_update(const __bf16* lds, int buf, const Frag2 (&qf)[TPW][2], int nown,
                                                float lscale, float (&mrun)[TPW], float (&lsum)[TPW],
                                                f32x4 (&acc)[TPW][4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const __bf16* kb = lds + buf * DMA_TILE;
  const __bf16* vb = lds + (DMA_NBUF + buf) * DMA_TILE;
  bool valid[8];
  if constexpr (MASK) {
    const uint8_t* mb = reinterpret_cast<const uint8_t*>(lds + 2 * DMA_NBUF * DMA_TILE) + 32 * buf;
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(mb + 16 * kst + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) valid[4 * kst + r] = ((w >> (8 * r)) & 0xffu) != 0;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) valid[e] = true;
  }
  Frag2 kf[2][2];
#pragma unroll
  for (int kst = 0; kst < 2; ++kst)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kst][ks].hi = *reinterpret_cast<const bf16x8*>(kb + swz(16 * kst + c16, 4 * ks + g));
  // V^T fragments by transposed reads: lane j of a 16-lane group points at
  // row kbase + j/4, channels dmap_run(dt, j%4) .. +3; lane i then holds
  // keys kbase .. kbase+3 of channel dmap(dt, i) (natural order).
  Frag2 vf[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int c0 = dmap_run<false>(dt, c16 & 3);
    const int r0 = 4 * g + (c16 >> 2);
    const int r1 = 16 + r0;
    const bf16x4 a = lds_read_tr(vb + r0 * HD + 8 * ((c0 >> 3) ^ (r0 & 7)) + (c0 & 7));
    const bf16x4 b = lds_read_tr(vb + r1 * HD + 8 * ((c0 >> 3) ^ (r1 & 7)) + (c0 & 7));
    vf[dt].hi = cat44(a, b);
  }
  kv_compute<1, TPW, MASK>(kf, vf, valid, qf, nown, lscale * LOG2E, mrun, lsum, acc);
}

// Stream key tiles [tile0, tile1) (all inside [0, n)) of one head.
template <int TPW, int NW, bool MASK, int KP = 1>
__device__ __forceinline__ void kv_stream_dma(const u16* __restrict__ K, const u16* __restrict__ V, long long st,
                                              const uint8_t* __restrict__ mask, int tile0, int tile1, float lscale,
                                              __bf16* lds, const Frag2 (&qf)[TPW][2], int nown, float (&mrun)[TPW],
                                              float (&lsum)[TPW], f32x4 (&acc)[TPW][4], int kp = 0) {
  constexpr int CNT = 8 / NW + (MASK ? 1 : 0);  // copies per tile and wave
  static_assert(DMA_DIST - KP <= 5, "wait_vmcnt_rt covers up to 5 tiles");
  // a tile's buffer is refilled only after the step that read it
  static_assert(DMA_DIST + KP <= DMA_NBUF, "ring too short for the copy distance");
  const int T = tile1 - tile0;
  for (int j = 0; j < DMA_DIST && j < T; ++j)
    dma_issue_tile<NW, MASK>(K, V, st, mask, (tile0 + j) * 32, lds, j % DMA_NBUF);
  // one step per KP tiles: the KP wave groups work on their tiles of the
  // step at the same time, between one barrier and the next
  for (int t = 0; t < T; t += KP) {
    wait_vmcnt_rt<CNT>(max(0, min(DMA_DIST - KP, T - t - KP)));
    barrier_only();
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (t + DMA_DIST + i < T)
        dma_issue_tile<NW, MASK>(K, V, st, mask, (tile0 + t + DMA_DIST + i) * 32, lds, (t + DMA_DIST + i) % DMA_NBUF);
    if (t + kp < T) dma_tile_update<TPW, MASK>(lds, (t + kp) % DMA_NBUF, qf, nown, lscale, mrun, lsum, acc);
  }
  barrier_only();
}

struct BvArgs {
  int BH;                   // heads (for the row-group block mapping)
  const void* k;
  const void* v;
  const uint8_t* key_mask;  // [B][n] or null
  const __bf16* qt_hi;      // [BH][M][d]
  const __bf16* qt_lo;
  float* pmax;              // [BH][S][M]
  float* psum;              // [BH][S][M]
  float* pacc;              // [BH][S][d/4][M][4]: 4-channel runs, each run's rows contiguous
  int n, H, S, tpc, ntiles;
  float lscale;             // d^-1/4 (Qt carries the other factor)
  Strides in;               // of k and v
};

// Waves of the B V / pseudo-inverse launch: one per 16 landmarks up to 128,
// four above (each then owning several landmark tiles).
template <int M>
constexpr int bv_waves() {
  return M <= 128 ? nwaves<M>() : 4;
}

// Row groups of the B V blocks.  With bf16 I/O at d = 64 and 128 landmarks,
// a B V block covers half of the landmark rows of its key chunk: two blocks
// per (head, chunk), each the 64-landmark block with a row offset, so the
// chunks can be twice as long for the same number of blocks and the
// partials that k_mw merges halve.  The two row groups of one chunk run on
// one XCD (their blocks are 8 apart), where its K and V tiles are fetched
// into L2 once.  At 256 landmarks the split does not pay: with four 64-row
// groups the live K and V tiles of an XCD outgrow its L2 (B V launch 35 ->
// 49 us at 1 x 4 x 65536, k_mw 19 -> 13 us), and two 128-row groups still
// lose 2 us over the two launches.
template <typename IO, int M, int D>
constexpr int bv_row_groups() {
  return bv_row_groups_for((int)sizeof(IO), M, D);
}
// Rows and waves of one B V block, and the waves of the whole launch.
template <typename IO, int M, int D>
constexpr int bv_rows() {
  return M / bv_row_groups<IO, M, D>();
}
template <typename IO, int M, int D>
constexpr int bv_launch_waves() {
  return bv_row_groups<IO, M, D>() > 1 ? nwaves<M>() : bv_waves<M>();
}

// Partial B V of one (head, key chunk): all M landmarks.  With NW waves
// and TM landmark tiles, wave w owns landmark tiles {w, w + NW, ...}; when
// there are twice as many waves as tiles (m <= 64) the tile's two waves
// take alternate key tiles (KP = 2), both tiles of a pair in the same
// barrier step, and fold their online-softmax states together in LDS at
// the end.
// LDS the KP = 2 fold of bv_block needs (floats: max, sum and D/4 channel
// values per lane of each of the TM waves).
template <int M, int D>
constexpr int bv_fold_bytes() {
  return 4 * (M / 16) * 64 * (2 + D / 4);
}

// MB landmark rows r0 .. r0 + MB - 1 of M (MB = M without row groups).
template <typename IO, int M, bool EDGE, int D = HD, int MB = M>
__device__ void bv_block(const BvArgs& a, int bh, int chunk, int r0, __bf16* lds) {
  constexpr int TM = MB / 16;
  constexpr int NW = bv_waves<MB>();
  constexpr int KP = (M <= 128 && NW % TM == 0) ? NW / TM : 1;
  constexpr int NWT = KP > 1 ? TM : NW;  // waves per key parity
  constexpr int TPW = (TM + NWT - 1) / NWT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wave = w % NWT, kp = w / NWT;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = bh / a.H;
  const IO* K = reinterpret_cast<const IO*>(a.k) + a.in.base(bh, a.H);
  const IO* V = reinterpret_cast<const IO*>(a.v) + a.in.base(bh, a.H);
  const long long st = a.in.t;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  const int nown = (kp < KP && wave < TM) ? (TM - wave + NWT - 1) / NWT : 0;

  Frag2 qf[TPW][D / 32];
  float mrun[TPW], lsum[TPW];
  f32x4 acc[TPW][D / 16];
#pragma unroll
  for (int o = 0; o < TPW; ++o) {
    const int lt = wave + NWT * o;
    mrun[o] = NEG_BIG;
    lsum[o] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[o][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (o < nown) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const size_t off = ((size_t)bh * M + r0 + 16 * lt + c16) * D + 32 * ks + 8 * g;
        qf[o][ks].hi = *reinterpret_cast<const bf16x8*>(a.qt_hi + off);
        // bf16 keys: one bf16 pass (hi plane) against exact bf16 operands
        if constexpr (IOTraits<IO>::NS == 3) qf[o][ks].lo = *reinterpret_cast<const bf16x8*>(a.qt_lo + off);
      }
    }
  }
  const int tile0 = chunk * a.tpc;
  const int tile1 = min(a.ntiles, tile0 + a.tpc);
  // the landmark fragments arrive before any K/V copy is issued, so the
  // copy pipeline below is never drained to wait for them
  wait_vmcnt<0>();
  if constexpr (sizeof(IO) == 2 && D == HD) {
    // whole 32-key tiles by DMA; a ragged last tile (n % 32 != 0) through
    // registers, which zero and mask the keys past n
    const int tfull = min(tile1, a.n / 32);
    if (mask != nullptr)
      kv_stream_dma<TPW, NW, true, KP>(K, V, st, mask, tile0, tfull, a.lscale, lds, qf, nown, mrun, lsum, acc, kp);
    else
      kv_stream_dma<TPW, NW, false, KP>(K, V, st, mask, tile0, tfull, a.lscale, lds, qf, nown, mrun, lsum, acc, kp);
    if constexpr (EDGE)
      if (tfull < tile1)
        kv_stream<IO, TPW, 64 * NW, KP>(K, V, st, a.n, mask, tfull, tile1, a.lscale, lds, qf, nown, mrun, lsum, acc,
                                        kp);
  } else {
    kv_stream<IO, TPW, 64 * NW, KP, D>(K, V, st, a.n, mask, tile0, tile1, a.lscale, lds, qf, nown, mrun, lsum, acc,
                                       kp);
  }
  if constexpr (KP == 2) {
    // fold the odd-tile waves' states into the even-tile waves (same lanes)
    float* st = reinterpret_cast<float*>(lds) + (size_t)wave * 64 * (2 + D / 4) + lane;
    if (kp == 1 && nown > 0) {
      st[0] = mrun[0];
      st[64] = lsum[0];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[64 * (2 + 4 * dt + r)] = acc[0][dt][r];
    }
    __syncthreads();
    if (kp == 0 && nown > 0) {
      const float m1 = st[0], l1 = st[64];
      const float mn = fmaxf(mrun[0], m1);
      const float a0 = fast_exp2(mrun[0] - mn), a1 = fast_exp2(m1 - mn);
      mrun[0] = mn;
      lsum[0] = lsum[0] * a0 + l1 * a1;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[0][dt][r] = acc[0][dt][r] * a0 + st[64 * (2 + 4 * dt + r)] * a1;
    }
  }
#pragma unroll
  for (int o = 0; o < TPW; ++o) {
    if (o >= nown || kp != 0) break;
    const int i = r0 + 16 * (wave + NWT * o) + c16;
    const float ls = sum_g(lsum[o]);
    const size_t row = ((size_t)bh * a.S + chunk) * M + i;
    if (g == 0) {
      a.pmax[row] = mrun[o];  // log2 units of the scaled logit
      a.psum[row] = ls;
    }
    // lane (c16, g) holds channels 16 dt + 4 g .. + 3 of row i: run 4 dt + g
    float* const pr = a.pacc + ((size_t)bh * a.S + chunk) * (D / 4) * M * 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(pr + ((size_t)(4 * dt + g) * M + i) * 4) =
          make_float4(acc[o][dt][0], acc[o][dt][1], acc[o][dt][2], acc[o][dt][3]);
  }
}

// Blocks [0, npinv) run the fused pseudo-inverse (one per head); the rest
// run B V partials for (head, chunk).  Dynamic LDS = max of the two.
// EDGE: some padding landmarks (m not a multiple of 32) or a ragged last
// key tile (n not a multiple of 32); the code for them is compiled only into
// this instance, so the common shapes pay nothing for it.
// F16: the pseudo-inverse encoding of bf16 I/O (single fp16 or split bf16
// products; pa.f16 must match).  Each encoding is its own instance, so the
// register allocation of one is not shaped by the other (with both in one
// kernel the 128-landmark instance spilled 51 VGPRs to scratch).
template <typename IO, int M, bool EDGE, int D = HD, bool F16 = false>
__global__ __launch_bounds__((64 * bv_launch_waves<IO, M, D>())) void k_pinv_bv(PinvArgs pa, BvArgs ba, int npinv) {
  extern __shared__ __align__(16) __bf16 lds_dyn[];
  if ((int)blockIdx.x < npinv) {
    if constexpr (M <= 128) {
      if constexpr (sizeof(IO) == 4)
        pinv_block_f32<M, EDGE>(pa, blockIdx.x, reinterpret_cast<float*>(lds_dyn));
      else
        pinv_block<M, F16, EDGE>(pa, blockIdx.x, reinterpret_cast<u16*>(lds_dyn));
    } else if constexpr (sizeof(IO) == 2 && D == HD && bv_launch_waves<IO, M, D>() == 4) {
      gram_rows_body<M, D>(pa.la, pa.gAT, pa.gA16, pa.colpart, pa.rowpart, blockIdx.x,
                           reinterpret_cast<char*>(lds_dyn));
    }
    return;
  }
  const int id = blockIdx.x - npinv;
  constexpr int RG = bv_row_groups<IO, M, D>();
  if constexpr (RG == 1) {
    bv_block<IO, M, EDGE, D>(ba, id / ba.S, id % ba.S, 0, lds_dyn);
  } else {
    // blocks 8 apart take the row groups of one (head, chunk)
    const int rg = (id / 8) % RG, rest = id % 8 + 8 * (id / (8 * RG));
    if (rest >= ba.BH * ba.S) return;  // grid rounding; whole workgroup, before any barrier
    constexpr int MB = bv_rows<IO, M, D>();
    bv_block<IO, M, EDGE, D, MB>(ba, rest / ba.S, rest % ba.S, MB * rg, lds_dyn);
  }
}

// ---------------------------------------------------------------------------
// Exact branch (m == n): flash-style attention over all keys, 64 queries per
// workgroup (16 per wave), then the convolution added in the same C tiles.

struct ExactArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* key_mask;
  const float* conv_w;  // [H][conv_k] or null
  int conv_k;           // odd taps, 1 .. 65
  void* out;
  int n, H;
  float lscale;  // 1 / sqrt(d)
  Strides in, out_s;  // of q, k, v and of out
};

constexpr int EXACT_WIN = 144;            // conv window rows for 64 queries
constexpr int EXACT_VWLD = EXACT_WIN + 8;

template <typename IO, int D = HD>
constexpr int exact_lds_bytes() {
  constexpr int NS = IOTraits<IO>::NS;
  constexpr int kv = KV<IO, D>::LDS_BYTES;
  constexpr int win = D * EXACT_VWLD * 2 * (NS == 3 ? 2 : 1);
  return kv > win ? kv : win;
}

template <typename IO, int D = HD>
__global__ __launch_bounds__(256) void k_exact(ExactArgs a) {
  extern __shared__ __align__(16) __bf16 lds_dyn[];
  constexpr int NS = IOTraits<IO>::NS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int q0 = blockIdx.x * 64;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + a.in.base(bh, a.H);
  const IO* K = reinterpret_cast<const IO*>(a.k) + a.in.base(bh, a.H);
  const IO* V = reinterpret_cast<const IO*>(a.v) + a.in.base(bh, a.H);
  const long long st = a.in.t;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;

  const int tok = q0 + 16 * wave + c16;
  Frag2 qf[1][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    float x[8];
    if (tok < a.n) {
      IOTraits<IO>::load8(Q + tok * st + 32 * ks + 8 * g, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    qf[0][ks] = make_frag<NS>(x);
  }
  float mrun[1] = {NEG_BIG}, lsum[1] = {0.f};
  f32x4 acc[1][D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ntiles = (a.n + KV<IO, D>::KT - 1) / KV<IO, D>::KT;
  kv_stream<IO, 1, 256, 1, D>(K, V, st, a.n, mask, 0, ntiles, a.lscale, lds_dyn, qf, 1, mrun, lsum, acc);
  const float ls = sum_g(lsum[0]);
  const float inv = ls > 0.f ? 1.0f / ls : 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[0][dt] *= inv;
  if (a.conv_w != nullptr) {
    __bf16* Vh = lds_dyn;
    __bf16* Vl = lds_dyn + D * EXACT_VWLD;
    stage_v_window<IO, D>(V, st, a.n, q0, EXACT_WIN, Vh, Vl, EXACT_VWLD);
    __syncthreads();
    Frag2 tap[3];
    conv_taps(a.conv_w + (size_t)h * a.conv_k, a.conv_k, tap);
    conv_tile<NS, false, D>(Vh, Vl, EXACT_VWLD, 16 * wave, tap, acc[0]);
  }
  if (tok < a.n)
    store_row16<IO, false, D, true>(reinterpret_cast<IO*>(a.out) + a.out_s.base(bh, a.H) + tok * a.out_s.t, acc[0]);
}

}  // namespace nys
