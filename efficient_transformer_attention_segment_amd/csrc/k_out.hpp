// Output pass: out = F W + conv(V), with F = softmax(Qs Kt^T).
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.4
// (kernel_1 F = softmax(Q against the key landmarks), n x m; the context is
// F times A^+ times B V) and section 2.6 (context += depthwise conv of V).
//
// k_out (float32 I/O, and bf16 I/O at head sizes other than 64): a
// workgroup covers 128 tokens of one head (4 waves x 2 tiles of 16; 64
// tokens at d = 128).  The key landmarks, the W^T fragments and a V window
// (tokens t0 - 32 .. t0 + tokens + 48) are staged in LDS once, through
// registers as bf16 hi/lo with V stored transposed (landmarks and fragments
// stay in L2 where LDS cannot hold them), with every wave's Q rows already
// loading as B fragments.  Per 16-token tile a wave:
//   forms S^T = Kt Q^T (m x 16) on the matrix cores,
//   takes the softmax down each column with the whole F row in registers
//   (m <= 256: no online rescaling needed),
//   accumulates O^T = W^T F^T, F used directly from the S^T C tiles,
//   adds the convolution as three banded Toeplitz products into the same
//   accumulators,
//   and stores d / 4 channels per lane.
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
  const float* conv_w;   // [H][conv_k] or null
  int conv_k;            // odd taps, 1 .. 65
  const __bf16* kt_hi;   // [BH][M][d]
  const __bf16* kt_lo;
  const __bf16* wf_hi;   // [BH][d/16][M/32][64][8]
  const __bf16* wf_lo;
  void* out;
  int n, H;
  int mr;                // landmarks of the method (M = mr rounded up to 32)
  float lscale;          // d^-1/4
  Strides in, out_s;     // of q and v, and of out
  int q_stream;          // bf16 output pass: read Q with streaming loads (0 when Q was just written)
};

// Logits of padding landmarks (16 it + 4g + r >= mr) -> -inf, in S^T tiles.
template <int TM>
__device__ __forceinline__ void pad_mask_rows(f32x4 (&sacc)[TM], int mr) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int it = 0; it < TM; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (16 * it + 4 * g + r >= mr) sacc[it][r] = -INFINITY;
}

// Tokens per workgroup (4 waves x U tiles of 16) and the V window rows
// (t0 - 32 .. t0 + TOK + 48) of the generic output pass.
template <typename IO, int M, int D>
struct OutLayout {
  static constexpr int NS = IOTraits<IO>::NS;
  static constexpr int TOK = D > 64 ? 64 : 128;
  static constexpr int U = TOK / 64;
  static constexpr int WIN = TOK + 80;
  static constexpr int VWLD = WIN + 8;
  static constexpr int KS = M / 32;
  static constexpr int KLD = D + 8;
  static constexpr int KT_ELEMS = M * KLD;                 // per part
  static constexpr int WF_ELEMS = (D / 16) * KS * 64 * 8;  // per part
  static constexpr int V_ELEMS = D * VWLD;                 // per part
  static constexpr int PARTS = NS == 3 ? 2 : 1;
  // the key landmarks, then the W^T fragments, are staged in LDS when they
  // fit the 160 KB beside the V window; otherwise they are read from global
  // memory (L2: every workgroup of the head reads the same data)
  static constexpr bool KT_LDS = 2 * PARTS * (KT_ELEMS + V_ELEMS) <= 160 * 1024;
  static constexpr bool WF_LDS = KT_LDS && 2 * PARTS * (KT_ELEMS + WF_ELEMS + V_ELEMS) <= 160 * 1024;
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_WF = OFF_KT + (KT_LDS ? PARTS * KT_ELEMS : 0);
  static constexpr int OFF_V = OFF_WF + (WF_LDS ? PARTS * WF_ELEMS : 0);
  static constexpr int TOTAL = OFF_V + PARTS * V_ELEMS;
  static constexpr int LDS_BYTES = TOTAL * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "k_out LDS");
};

// grid (ceil(n / TOK), BH), block 256, dynamic LDS OutLayout::LDS_BYTES.
template <typename IO, int M, bool PAD, int D = HD>
__global__ __launch_bounds__(256) void k_out(OutArgs a) {
  extern __shared__ __align__(16) __bf16 lds_dyn[];
  using Ly = OutLayout<IO, M, D>;
  constexpr int NS = Ly::NS, KS = Ly::KS, TM = M / 16, DK = D / 32, DT = D / 16, U = Ly::U;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, h = bh % a.H;
  const int t0 = blockIdx.x * Ly::TOK;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + a.in.base(bh, a.H);
  const IO* V = reinterpret_cast<const IO*>(a.v) + a.in.base(bh, a.H);
  const long long st = a.in.t;

  const __bf16* const ksh = a.kt_hi + (size_t)bh * M * D;
  const __bf16* const ksl = a.kt_lo + (size_t)bh * M * D;
  __bf16* const kth_lds = lds_dyn + Ly::OFF_KT;
  __bf16* const ktl_lds = kth_lds + Ly::KT_ELEMS;
  const __bf16* const kth = Ly::KT_LDS ? kth_lds : ksh;
  const __bf16* const ktl = Ly::KT_LDS ? ktl_lds : ksl;
  constexpr int KROW = Ly::KT_LDS ? Ly::KLD : D;
  const __bf16* const wsh = a.wf_hi + (size_t)bh * Ly::WF_ELEMS;
  const __bf16* const wsl = a.wf_lo + (size_t)bh * Ly::WF_ELEMS;
  __bf16* const wfh_lds = lds_dyn + Ly::OFF_WF;
  __bf16* const wfl_lds = wfh_lds + Ly::WF_ELEMS;
  const __bf16* const wfh = Ly::WF_LDS ? wfh_lds : wsh;
  const __bf16* const wfl = Ly::WF_LDS ? wfl_lds : wsl;
  __bf16* vh = lds_dyn + Ly::OFF_V;
  __bf16* vl = vh + Ly::V_ELEMS;

  // ---- stage Kt, W^T fragments and the V window
  {
    if constexpr (Ly::KT_LDS) {
      for (int idx = threadIdx.x; idx < M * (D / 8); idx += 256) {
        const int row = idx / (D / 8), cc = idx % (D / 8);
        *reinterpret_cast<bf16x8*>(kth_lds + row * Ly::KLD + 8 * cc) =
            *reinterpret_cast<const bf16x8*>(ksh + (size_t)row * D + 8 * cc);
        if constexpr (NS == 3)
          *reinterpret_cast<bf16x8*>(ktl_lds + row * Ly::KLD + 8 * cc) =
              *reinterpret_cast<const bf16x8*>(ksl + (size_t)row * D + 8 * cc);
      }
    }
    if constexpr (Ly::WF_LDS) {
      for (int idx = threadIdx.x; idx < Ly::WF_ELEMS / 8; idx += 256) {
        *reinterpret_cast<bf16x8*>(wfh_lds + 8 * idx) = *reinterpret_cast<const bf16x8*>(wsh + 8 * idx);
        if constexpr (NS == 3)
          *reinterpret_cast<bf16x8*>(wfl_lds + 8 * idx) = *reinterpret_cast<const bf16x8*>(wsl + 8 * idx);
      }
    }
    if (a.conv_w != nullptr) stage_v_window<IO, D>(V, st, a.n, t0, Ly::WIN, vh, vl, Ly::VWLD);
  }
  // Q B fragments of the wave's tiles, in flight with the staging copies
  Frag2 qf2[U][DK];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ts = t0 + 16 * U * wave + 16 * u;
    const int tok = min(ts + c16, a.n - 1);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      float x[8];
      IOTraits<IO>::load8(Q + tok * st + 32 * ks + 8 * g, x);
      qf2[u][ks] = make_frag<NS>(x);
    }
  }
  Frag2 tap[3];
  if (a.conv_w != nullptr) conv_taps(a.conv_w + (size_t)h * a.conv_k, a.conv_k, tap);
  __syncthreads();

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ts = t0 + 16 * U * wave + 16 * u;  // tile start
    if (ts >= a.n) continue;
    const int tok = ts + c16;
    const Frag2(&qf)[DK] = qf2[u];
    // S^T = Kt Q^T: sacc[it][r] = logit(tok, landmark 16 it + 4g + r)
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
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8] = {sacc[2 * ks][0] * inv,     sacc[2 * ks][1] * inv,     sacc[2 * ks][2] * inv,
                    sacc[2 * ks][3] * inv,     sacc[2 * ks + 1][0] * inv, sacc[2 * ks + 1][1] * inv,
                    sacc[2 * ks + 1][2] * inv, sacc[2 * ks + 1][3] * inv};
      const Frag2 pf = make_frag<NS>(x);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        Frag2 wf;
        const int off = ((dt * KS + ks) * 64 + lane) * 8;
        wf.hi = *reinterpret_cast<const bf16x8*>(wfh + off);
        if constexpr (NS == 3) wf.lo = *reinterpret_cast<const bf16x8*>(wfl + off);
        oacc[dt] = mma<NS>(wf, pf, oacc[dt]);
      }
    }
    if (a.conv_w != nullptr) conv_tile<NS, false, D>(vh, vl, Ly::VWLD, ts - t0, tap, oacc);
    if (tok < a.n)
      store_row16<IO, false, D, true>(reinterpret_cast<IO*>(a.out) + a.out_s.base(bh, a.H) + tok * a.out_s.t, oacc);
  }
}

// ---------------------------------------------------------------------------
// bf16 I/O: persistent, pipelined output pass.  A workgroup owns a
// contiguous token range of one head and walks it in units of 64 tokens (one
// 16-token tile per wave).  The key landmarks, the W^T fragments and the
// conv taps are loaded once per workgroup.  V streams through a ring of four
// 64-row groups in LDS (absolute token row r at ring row r & 255): during
// unit u the workgroup writes group u / 64 + 2 (loaded into registers during
// the previous unit) into the slot that unit last read, and loads group
// u / 64 + 3; each unit's Q rows load into registers two units ahead.  Only
// ordinary loads feed the loop, so the compiler's waits track exactly the
// registers each step needs and the output stores stay in flight across
// units.  48 KB of LDS at m = 64 lets three workgroups share a CU.
//
// Ring layout: row r has its 16-byte chunk c at chunk position c ^ (2 (r & 3)),
// so the four rows of one transposed conv read fall on different bank halves,
// and rows with bit 3 set keep the two 8-byte halves of each chunk swapped,
// so the rows r and r + 8 that two lane groups read in the same cycle fall on
// different banks too.  The key landmarks sit in LDS with their 16-byte chunks
// XOR-swizzled by (row / 2) % 8, which spreads the 16 rows of a fragment read
// over all 64 banks.
// Each lane's conv reads sit at a fixed row offset from the unit's first token,
// so their addresses are a per-unit row term plus per-lane constants.

// A workgroup of NW waves (4, or 8 where LDS allows only one workgroup per
// CU) takes units of 16 NW tokens, one 16-token tile per wave; the V ring
// holds four units' rows.
template <int NW>
constexpr int outs_unit() {
  return 16 * NW;  // tokens per unit (and rows per ring group)
}
template <int NW>
constexpr int outs_ring() {
  return 4 * outs_unit<NW>();  // ring rows (4 groups)
}
constexpr int OUTS_UNIT = outs_unit<4>();

// The wave count of the persistent output pass: 8 above 192 landmarks (the
// landmarks and W^T fragments alone take 64 KB, so one workgroup per CU: 8
// waves hide twice the latency of 4, 42 -> 38 us at 1 x 4 x 65536, m = 256),
// otherwise 4 (several workgroups per CU; 8 waves there were slower, 19.5 ->
// 25.6 us at 4 x 12 x 4096, m = 64).
template <int M>
constexpr int outs_waves() {
  return M > 192 ? 8 : 4;
}

template <int M, int NW = 4>
struct OutStreamLayout {
  static constexpr int KS = M / 32;
  static constexpr int KT_ELEMS = M * HD;
  static constexpr int WF_ELEMS = 4 * KS * 64 * 8;
  static constexpr int RING_ELEMS = outs_ring<NW>() * HD;
  static constexpr int LDS_BYTES = 2 * (KT_ELEMS + WF_ELEMS + RING_ELEMS);
};

template <int NW>
__device__ __forceinline__ int vring_pos(int r, int chunk) {
  return (r & (outs_ring<NW>() - 1)) * HD + 8 * (chunk ^ (2 * (r & 3)));
}

// One group in flight through registers: thread t holds 32 bytes of row
// UNIT G + t / 4 (16-byte chunks 2 (t % 4) and 2 (t % 4) + 1); zero outside [0, n).
struct VGroup {
  uint4 x[2];
};
template <int NW>
__device__ __forceinline__ void vgroup_load(const u16* V, long long st, int n, int G, VGroup& b) {
  const int t = threadIdx.x;
  const int r = outs_unit<NW>() * G + (t >> 2);
  if (r >= 0 && r < n) {
    const uint4* src = reinterpret_cast<const uint4*>(V + r * st) + 2 * (t & 3);
    if constexpr (NW == 8) {
      // 8-wave units (above 192 landmarks): streaming loads measured faster
      // (n = 65536: 184 -> 181 us per call); at 4 waves they were slower
      const u32x4 x0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      const u32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + 1);
      b.x[0] = make_uint4(x0[0], x0[1], x0[2], x0[3]);
      b.x[1] = make_uint4(x1[0], x1[1], x1[2], x1[3]);
    } else {
      b.x[0] = src[0];
      b.x[1] = src[1];
    }
  } else {
    b.x[0] = b.x[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}
template <int NW>
__device__ __forceinline__ void vgroup_store(const VGroup& b, int G, __bf16* ring) {
  const int t = threadIdx.x;
  const int r = outs_unit<NW>() * G + (t >> 2);
  // rows with bit 3 set keep the two 8-byte halves of each chunk swapped, so
  // that the transposed reads of rows r and r + 8 (lane groups 0 and 1 of
  // one read) fall in different banks
  const bool sw = (r >> 3) & 1;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint4 v = b.x[c];
    *reinterpret_cast<uint4*>(ring + vring_pos<NW>(r, 2 * (t & 3) + c)) = sw ? make_uint4(v.z, v.w, v.x, v.y) : v;
  }
}

// Per-lane constants of the conv reads of the wave's tile: read (kk, half, dt)
// of the unit starting at token t0 is at ring row (t0 + rel[kk][half]) & 255,
// element offset coff[kk][half][dt] within that row.
struct ConvLane {
  int rel[3][2];
  int coff[3][2][4];
};
__device__ __forceinline__ void conv_lane_init(ConvLane& cl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int rel = 16 * wave - HALO + 32 * kk + 8 * g + (c16 >> 2) + 4 * half;
      cl.rel[kk][half] = rel;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c0 = dmap_run<true>(dt, c16 & 3);
        // rel & 3 == row & 3 and rel & 8 == row & 8 (rows differ from rel by a multiple of 64)
        cl.coff[kk][half][dt] = 8 * ((c0 >> 3) ^ (2 * (rel & 3))) + ((c0 & 7) ^ (4 * ((rel >> 3) & 1)));
      }
    }
}

// Convolution of the wave's 16-token tile of the unit starting at t0 from
// the ring (window rows ts - 32 .. ts + 63 in three 32-row steps; taps beyond
// the 80 needed are 0).
template <int NW>
__device__ __forceinline__ void conv_tile_ring(const __bf16* ring, int t0, const ConvLane& cl, const Frag2 (&tap)[3],
                                               f32x4 (&oacc)[4]) {
  constexpr int RING = outs_ring<NW>();
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    const __bf16* r0 = ring + ((t0 + cl.rel[kk][0]) & (RING - 1)) * HD;
    const __bf16* r1 = ring + ((t0 + cl.rel[kk][1]) & (RING - 1)) * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x4 x0 = lds_read_tr(r0 + cl.coff[kk][0][dt]);
      const bf16x4 x1 = lds_read_tr(r1 + cl.coff[kk][1][dt]);
      const bf16x8 vh = cat44(x0, x1);
      oacc[dt] = mfma(vh, tap[kk].hi, oacc[dt]);
      oacc[dt] = mfma(vh, tap[kk].lo, oacc[dt]);
    }
  }
}

// Q rows are read here for the last time in the call: streaming loads
// (stream != 0), so they do not displace what this pass and the call still
// re-read (V, W, Kt).  The module's q, written by its projection just
// before, is read with ordinary loads.
__device__ __forceinline__ void load_q16(const u16* Q, long long st, int n, int tok, bf16x8 (&qf)[2], int stream) {
  const int g = (threadIdx.x & 63) >> 4;
  const u16* row = Q + min(tok, n - 1) * st + 8 * g;
  if (stream) {
    qf[0] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(row));
    qf[1] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(row + 32));
  } else {
    qf[0] = *reinterpret_cast<const bf16x8*>(row);
    qf[1] = *reinterpret_cast<const bf16x8*>(row + 32);
  }
}

// grid (blocks per head, B H), 256 threads; workgroup x covers tokens
// [x R, min(n, (x + 1) R)), R a multiple of 64.  junk: >= 16 * 64 bf16, the
// destination of tiles past the range.  Two Q register buffers alternate
// between even and odd units (loaded two units before use).
template <int M, bool CONV, bool PAD, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_out_stream(OutArgs a, int R, u16* junk) {
  constexpr int OUTS_UNIT = outs_unit<NW>();
  using Ly = OutStreamLayout<M, NW>;
  constexpr int KS = Ly::KS, TM = M / 16;
  __shared__ __align__(16) __bf16 kt_s[Ly::KT_ELEMS];
  __shared__ __align__(16) __bf16 wf_s[Ly::WF_ELEMS];
  __shared__ __align__(16) __bf16 ring[CONV ? Ly::RING_ELEMS : 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // XCD-aware placement: workgroup i of the launch runs on XCD i mod 8, so
  // when the head count is a multiple of 8 the linear index is remapped to
  // put every range of a head on one XCD (its landmark and W^T fragments,
  // and the V rows neighbouring ranges share, then come into one L2)
  int by = blockIdx.y, bx = blockIdx.x;
  if ((gridDim.y & 7) == 0) {
    const int L = blockIdx.x + blockIdx.y * gridDim.x, s = L >> 3;
    by = (L & 7) + 8 * (s / gridDim.x);
    bx = s % gridDim.x;
  }
  const int bh = by, h = bh % a.H;
  const int tb = bx * R;
  const int te = min(a.n, tb + R);
  const int nunits = (te - tb + OUTS_UNIT - 1) / OUTS_UNIT;
  const u16* Q = reinterpret_cast<const u16*>(a.q) + a.in.base(bh, a.H);
  const u16* V = reinterpret_cast<const u16*>(a.v) + a.in.base(bh, a.H);
  u16* O = reinterpret_cast<u16*>(a.out) + a.out_s.base(bh, a.H);
  const long long st = a.in.t, ot = a.out_s.t;

  // ---- prologue: landmarks and W^T fragments (DMA), V groups G0 - 1 .. G0 + 1
  // (through registers), group G0 + 2 and the Q rows of units 0, 1 in flight
  {
    const __bf16* kt = a.kt_hi + (size_t)bh * M * HD;
    const __bf16* wf = a.wf_hi + (size_t)bh * 4 * KS * 64 * 8;
    const int rsub = lane >> 3;
    for (int c = wave; c < M / 8; c += NW) {
      const int row = 8 * c + rsub;
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      dma16(kt + (size_t)row * HD + 8 * chunk, kt_s + 8 * c * HD);
    }
    for (int c = wave; c < 4 * KS; c += NW) dma16(wf + (size_t)c * 512 + 8 * lane, wf_s + 512 * c);
  }
  const int G0 = tb / OUTS_UNIT;
  const int Glast = G0 + nunits;  // last group any unit reads (rows up to the range end + 32)
  VGroup vb;
  ConvLane cl;
  if constexpr (CONV) {
    VGroup pre[3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (G0 - 1 + i <= Glast) vgroup_load<NW>(V, st, a.n, G0 - 1 + i, pre[i]);
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (G0 - 1 + i <= Glast) vgroup_store<NW>(pre[i], G0 - 1 + i, ring);
    if (G0 + 2 <= Glast) vgroup_load<NW>(V, st, a.n, G0 + 2, vb);
    conv_lane_init(cl);
  }
  bf16x8 qb[2][2];
  load_q16(Q, st, a.n, tb + 16 * wave + c16, qb[0], a.q_stream);
  if (nunits > 1) load_q16(Q, st, a.n, tb + OUTS_UNIT + 16 * wave + c16, qb[1], a.q_stream);
  Frag2 tap[3];
  if constexpr (CONV) conv_taps(a.conv_w + (size_t)h * a.conv_k, a.conv_k, tap);
  wait_vmcnt<0>();  // the landmark / fragment copies (the register loads are tracked by the compiler)
  __syncthreads();

  const float ls2 = a.lscale * LOG2E;
  auto unit = [&](int u, bf16x8(&q)[2]) {
    const int t0 = tb + OUTS_UNIT * u;
    const int G = t0 / OUTS_UNIT;
    if (u > 0) __syncthreads();  // last unit's ring writes are visible; its reads of the slot reused below are done
    if constexpr (CONV) {
      if (G + 2 <= Glast) vgroup_store<NW>(vb, G + 2, ring);  // slot of G - 2: last read by the previous unit
      if (G + 3 <= Glast) vgroup_load<NW>(V, st, a.n, G + 3, vb);
    }
    const int ts = t0 + 16 * wave;
    // S^T = Kt Q^T: sacc[it][r] = logit(token ts + c16, landmark 16 it + 4g + r)
    f32x4 sacc[TM];
#pragma unroll
    for (int it = 0; it < TM; ++it) {
      sacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kr = 16 * it + c16;  // chunks XOR-swizzled by (row / 2) % 8: 16 rows, 64 distinct banks
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt_s + kr * HD + 8 * ((4 * ks + g) ^ ((kr >> 1) & 7)));
        sacc[it] = mfma(kf, q[ks], sacc[it]);
      }
    }
    if (u + 2 < nunits) load_q16(Q, st, a.n, t0 + 2 * OUTS_UNIT + 16 * wave + c16, q, a.q_stream);  // unit u + 2
    if constexpr (PAD) pad_mask_rows(sacc, a.mr);
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[it][r]);
    mx = max_g(mx);
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
      const f32x8 pv = {sacc[2 * ks][0] * inv,     sacc[2 * ks][1] * inv,     sacc[2 * ks][2] * inv,
                        sacc[2 * ks][3] * inv,     sacc[2 * ks + 1][0] * inv, sacc[2 * ks + 1][1] * inv,
                        sacc[2 * ks + 1][2] * inv, sacc[2 * ks + 1][3] * inv};
      const bf16x8 pf = __builtin_convertvector(pv, bf16x8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 wf = *reinterpret_cast<const bf16x8*>(wf_s + ((dt * KS + ks) * 64 + lane) * 8);
        oacc[dt] = mfma(wf, pf, oacc[dt]);
      }
    }
    if constexpr (CONV) conv_tile_ring<NW>(ring, t0, cl, tap, oacc);
    u16* dst = ts + c16 < te ? O + (ts + c16) * ot : junk + c16 * HD;
    store_row16<u16, true, HD, true>(dst, oacc);
  };
  int u = 0;
  for (; u + 1 < nunits; u += 2) {
    unit(u, qb[0]);
    unit(u + 1, qb[1]);
  }
  if (u < nunits) unit(u, qb[0]);
}

}  // namespace nys
