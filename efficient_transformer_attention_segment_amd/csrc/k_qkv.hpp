// The self-attention module's q/k/v projection: y = x W^T + b.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.2: q,
// k and v come from three linear projections of the hidden states (the
// query, key and value weights, stacked here as one [3 H d, hidden] matrix
// in nn.Linear's [out, in] layout), split into heads.
//
// x [rows][K] and W [N][K] are both K-contiguous, so every matrix-core
// operand is a 16-byte run of one row.
//
// k_qkv_bf16: 128 x 128 output tiles, 4 waves of 64 x 64 (three workgroups
//   per CU), the contraction in steps of 64: each step's tiles are stored
//   from registers into one LDS stage (rows of 128 bytes, 16-byte chunks
//   XOR-swizzled by (row / 2) & 7 so the fragment reads of 16 rows hit
//   distinct banks) while the next step's tiles load into registers;
//   LDS-only barriers, so those loads stay in flight across them.  Each
//   wave forms the transposed tile, y^T = W x^T, on v_mfma_f32_16x16x32_bf16,
//   so a lane holds 4 consecutive output columns of one row: the bias is
//   added in float32, and the wave's 64 x 64 bf16 block is staged in LDS and
//   stored as whole 128-byte rows (16 bytes per lane).  Every XCD walks its
//   own row tiles first for each column tile (qkv_tile).
// k_qkv_f32: float32 I/O on the float32 matrix core (v_mfma_f32_16x16x4f32),
//   64 x 64 tiles, register-staged float32 LDS tiles, for float32 accuracy.
#pragma once

#include "common.hpp"

namespace nys {

// Landmarks formed in the bf16 projection's epilogue (section 2.3 of the
// same page: each landmark is the mean of n / m contiguous scaled q or k
// rows).  Used when d = 64, the landmark count is a multiple of 32 and the
// segment length L = n / m divides 64: every wave's 64 output rows then hold
// whole segments of one sequence, and its 64 output columns are one head's
// q, k or v channels.  The wave sums, per segment, the bf16 values it
// stores (what the landmark pass would read back) in float32, scales by
// d^-1/4 / L and writes the landmark rows as the landmark pass does (float32
// and the bf16 hi/lo split); workgroup 0 also clears the meeting slots.
// (QkvLandmarks, the landmark targets, is declared in common.hpp for the
// host side too.)

struct QkvArgs {
  const void* x;     // [rows][K]
  const void* w;     // [N][K]
  const void* bias;  // [N] or null
  void* y;           // [rows][N]
  int rows, N, K;
  int fold;          // bf16 only: form the landmarks (lm) in the epilogue
  QkvLandmarks lm;
};

constexpr int QB_BM = 128, QB_BN = 128, QB_BK = 64, QB_NT = 256;
constexpr int QB_ATILE = QB_BM * QB_BK, QB_BTILE = QB_BN * QB_BK;  // bf16 elements
// output staging after the contraction: each wave's 64 x 64 bf16 block with
// row stride QB_SLD (144 bytes, so the 16 rows of a fragment store start on
// distinct banks), in the LDS the tile stage used (every wave has passed its
// last read of it)
constexpr int QB_SLD = 72;
constexpr int QB_LDS_TILES = (QB_ATILE + QB_BTILE) * 2;  // bytes: one stage
constexpr int QB_LDS_OUT = (QB_NT / 64) * 64 * QB_SLD * 2;
constexpr int QB_LDS = QB_LDS_TILES > QB_LDS_OUT ? QB_LDS_TILES : QB_LDS_OUT;

// Tiles (tm, tn) of a launch: linear index L runs on XCD L % 8; XCD x takes
// the row tiles x, x + 8, ... and walks them first for each column tile, so
// its x panels (a few MB) stay in its L2 while the W tiles stream past (the
// other order keeps all of W live beside the panels and overflows the L2).
__host__ __device__ inline int qkv_grid(int rows, int N, int BM, int BN) {
  const int tm = (rows + BM - 1) / BM, tn = (N + BN - 1) / BN;
  return 8 * tn * ((tm + 7) / 8);
}
__device__ __forceinline__ void qkv_tile(int rows, int N, int BM, int BN, int& tm, int& tn) {
  const int L = blockIdx.x, xcd = L & 7, s = L >> 3;
  const int mx = ((rows + BM - 1) / BM + 7) / 8;  // row tiles per XCD
  tn = s / mx;
  tm = xcd + 8 * (s % mx);
  (void)N;
}

// Tile rows of 64 bf16 (128 bytes) with 16-byte chunk c of row r at chunk
// position c ^ ((r >> 1) & 7): the 16 rows of one fragment read (two
// parities x eight positions) then cover all 64 banks.
__device__ __forceinline__ int qswz(int row, int chunk) {
  if constexpr (QB_BK == 128)
    return row * QB_BK + 8 * (chunk ^ (row & 15));  // 256-byte rows: 16 positions per row
  else
    return row * QB_BK + 8 * (chunk ^ ((row >> 1) & 7));
}

// Sum of v over aligned groups of G lanes within each 16-lane row (G = 1,
// 2, 4, 8 or 16; every lane of a group gets the group's sum).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<DPP_QUAD_1032>(v);
  if constexpr (G >= 4) v += dpp<DPP_QUAD_2301>(v);
  if constexpr (G >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}

// The landmark rows of one wave's 64 x 64 output block (rows r0 .. r0 + 63,
// columns c0 .. c0 + 63) from its stored bf16 values yv[j][i] (lane: row
// r0 + 16 i + lane % 16, columns c0 + 16 j + 4 (lane / 16) + 0..3).  L:
// segment length (divides 64).  Segments of L rows: for L >= 16 the sum over
// L / 16 row tiles in registers, then over the 16 lanes of a row; for
// L < 16 over groups of L lanes.  Fixed order, so deterministic.
template <int L>
__device__ __forceinline__ void qkv_landmarks(const QkvLandmarks& lm, const uint2 (&yv)[4][4], int r0, int c0,
                                              int rows, int N) {
  const int hd = lm.H * HD;
  if (c0 >= N || r0 >= rows) return;
  const int which = c0 / hd;  // 0: q, 1: k, 2: v (no landmarks)
  if (which >= 2) return;
  const int h = (c0 - which * hd) / HD;
  const int b = r0 / lm.n, t0 = r0 - b * lm.n;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  float* const dst = which == 0 ? lm.qt : lm.kt;
  __bf16* const dhi = which == 0 ? lm.qt_hi : lm.kt_hi;
  __bf16* const dlo = which == 0 ? lm.qt_lo : lm.kt_lo;
  const size_t head = (size_t)(b * lm.H + h) * lm.m;
  constexpr int TI = L >= 16 ? L / 16 : 1;  // row tiles per segment
  constexpr int GL = L >= 16 ? 16 : L;      // lanes per segment within a row tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i0 = 0; i0 < 4; i0 += TI) {
      float sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = i0; i < i0 + TI; ++i) {
        sv[0] += bf16u_to_f32(yv[j][i].x & 0xffffu);
        sv[1] += bf16u_to_f32(yv[j][i].x >> 16);
        sv[2] += bf16u_to_f32(yv[j][i].y & 0xffffu);
        sv[3] += bf16u_to_f32(yv[j][i].y >> 16);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = group_sum<GL>(sv[e]) * lm.scale;
      if (c16 % GL == 0) {
        const int l = (t0 + 16 * i0 + c16) / L;  // landmark
        const size_t o = (head + l) * HD + 16 * j + 4 * g;
        *reinterpret_cast<float4*>(dst + o) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        __bf16 hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split1(sv[e], hi[e], lo[e]);
        *reinterpret_cast<uint2*>(dhi + o) = make_uint2(__builtin_bit_cast(uint32_t, bf16x2{hi[0], hi[1]}),
                                                        __builtin_bit_cast(uint32_t, bf16x2{hi[2], hi[3]}));
        *reinterpret_cast<uint2*>(dlo + o) = make_uint2(__builtin_bit_cast(uint32_t, bf16x2{lo[0], lo[1]}),
                                                        __builtin_bit_cast(uint32_t, bf16x2{lo[2], lo[3]}));
      }
    }
  }
}

// grid qkv_grid(rows, N, QB_BM, QB_BN), QB_NT threads (waves of 64 x 64,
// QB_BM / 64 along the rows), dynamic LDS QB_LDS (one stage: the next step's
// tiles wait in registers while this step's are multiplied).
__global__ __launch_bounds__(QB_NT) void k_qkv_bf16(QkvArgs a) {
  extern __shared__ __align__(16) __bf16 qb_lds[];
  int tm, tn;
  qkv_tile(a.rows, a.N, QB_BM, QB_BN, tm, tn);
  if (tm * QB_BM >= a.rows) return;  // whole workgroup, before any barrier
  const int m0 = tm * QB_BM, n0 = tn * QB_BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  constexpr int WMS = QB_BM / 64;  // waves along the rows
  const int wm = wave % WMS, wn = wave / WMS;  // the wave's 64 x 64 part
  const u16* X = static_cast<const u16*>(a.x);
  const u16* Wt = static_cast<const u16*>(a.w);
  const int nk = (a.K + QB_BK - 1) / QB_BK;
  __bf16* const At = qb_lds;
  __bf16* const Bt = qb_lds + QB_ATILE;
  // per thread: QA 16-byte chunks of the A tile and QBn of the B tile
  constexpr int QA = QB_ATILE / 8 / QB_NT, QBn = QB_BTILE / 8 / QB_NT;
  uint4 ra[QA], rb[QBn];
  auto load = [&](int ks) {
    const int k0 = ks * QB_BK;
#pragma unroll
    for (int u = 0; u < QA; ++u) {
      const int idx = tid + QB_NT * u, row = idx / (QB_BK / 8), ch = idx % (QB_BK / 8);
      const int gr = m0 + row, gk = k0 + 8 * ch;
      ra[u] = (gr < a.rows && gk < a.K) ? *reinterpret_cast<const uint4*>(X + (size_t)gr * a.K + gk)
                                        : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < QBn; ++u) {
      const int idx = tid + QB_NT * u, row = idx / (QB_BK / 8), ch = idx % (QB_BK / 8);
      const int gr = n0 + row, gk = k0 + 8 * ch;
      rb[u] = (gr < a.N && gk < a.K) ? *reinterpret_cast<const uint4*>(Wt + (size_t)gr * a.K + gk)
                                     : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < QA; ++u) {
      const int idx = tid + QB_NT * u;
      *reinterpret_cast<uint4*>(At + qswz(idx / (QB_BK / 8), idx % (QB_BK / 8))) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < QBn; ++u) {
      const int idx = tid + QB_NT * u;
      *reinterpret_cast<uint4*>(Bt + qswz(idx / (QB_BK / 8), idx % (QB_BK / 8))) = rb[u];
    }
  };
  // the bias of the lane's output columns, loaded here so that it arrives
  // during the contraction (loaded in the epilogue, each load's round trip
  // would end the tile)
  const u16* const bias = static_cast<const u16*>(a.bias);
  uint2 bq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 64 * wn + 16 * j + 4 * g;
    bq[j] = (bias != nullptr && n < a.N) ? *reinterpret_cast<const uint2*>(bias + n) : make_uint2(0u, 0u);
  }
  f32x4 acc[4][4];  // [n subtile j][m subtile i]: y^T tiles
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS-only barriers: a fence would also drain the next step's loads
  load(0);
  for (int ks = 0; ks < nk; ++ks) {
    store();
    wait_lgkm0();
    barrier_only();
    if (ks + 1 < nk) load(ks + 1);  // in flight while this step is multiplied
#pragma unroll
    for (int kh = 0; kh < QB_BK / 32; ++kh) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(At + qswz(64 * wm + 16 * i + c16, 4 * kh + g));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bt + qswz(64 * wn + 16 * j + c16, 4 * kh + g));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mfma(bfr[j], af[i], acc[j][i]);
    }
    wait_lgkm0();
    barrier_only();  // every wave has read the tiles before the next store
  }

  // lane holds y[m][n .. n + 3] with m = m0 + 64 wm + 16 i + c16 and
  // n = n0 + 64 wn + 16 j + 4 g
  u16* const Y = static_cast<u16*>(a.y);
  // the wave's block goes through LDS (every wave is past the last read of
  // the tile stage) so that the stores below write whole 128-byte rows.
  // Measured at 16384 x 2304 x 768: the output stores cost about 17 us when
  // written as 8-byte pieces of each row (four stores per line) and about
  // 5 us as whole rows, with bit-identical results
  u16* const stg = reinterpret_cast<u16*>(qb_lds) + wave * (64 * QB_SLD);
  uint2 yv[4][4];  // [j][i]: the stored bf16 values (kept for the landmarks)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float b4[4] = {bf16u_to_f32(bq[j].x & 0xffffu), bf16u_to_f32(bq[j].x >> 16),
                         bf16u_to_f32(bq[j].y & 0xffffu), bf16u_to_f32(bq[j].y >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = acc[j][i];
      yv[j][i] = make_uint2(pack_bf16x2(v[0] + b4[0], v[1] + b4[1]), pack_bf16x2(v[2] + b4[2], v[3] + b4[3]));
      *reinterpret_cast<uint2*>(stg + (16 * i + c16) * QB_SLD + 16 * j + 4 * g) = yv[j][i];
    }
  }
  wait_lgkm0();
  // lane l: row l / 8 + 8 s of the block, 16 bytes at column 8 (l % 8)
#pragma unroll
  for (int sidx = 0; sidx < 8; ++sidx) {
    const int r = lane / 8 + 8 * sidx, c8 = lane % 8;
    const uint4 val = *reinterpret_cast<const uint4*>(stg + r * QB_SLD + 8 * c8);
    const int m = m0 + 64 * wm + r, n = n0 + 64 * wn + 8 * c8;
    if (m < a.rows) {
      u16* const dst = Y + (size_t)m * a.N + n;
      if (n + 8 <= a.N)
        *reinterpret_cast<uint4*>(dst) = val;
      else if (n < a.N)  // N is a multiple of 4 (16-byte rows of 3 H d)
        *reinterpret_cast<uint2*>(dst) = make_uint2(val.x, val.y);
    }
  }
  if (a.fold) {
    if (blockIdx.x == 0)
      for (int t = threadIdx.x; t < 2 * a.lm.H * (a.rows / a.lm.n); t += QB_NT) a.lm.slots[t] = 0ull;
    switch (a.lm.L) {
      case 2: qkv_landmarks<2>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      case 4: qkv_landmarks<4>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      case 8: qkv_landmarks<8>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      case 16: qkv_landmarks<16>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      case 32: qkv_landmarks<32>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      case 64: qkv_landmarks<64>(a.lm, yv, m0 + 64 * wm, n0 + 64 * wn, a.rows, a.N); break;
      default: break;
    }
  }
}

// ---------------------------------------------------------------- float32 ---
constexpr int QF_BM = 64, QF_BN = 64, QF_BK = 32, QF_LD = QF_BK + 4;

// grid qkv_grid(rows, N, 64, 64), 256 threads (4 waves of 32 x 32).
__global__ __launch_bounds__(256) void k_qkv_f32(QkvArgs a) {
  __shared__ __align__(16) float As[QF_BM * QF_LD];
  __shared__ __align__(16) float Bs[QF_BN * QF_LD];
  int tm, tn;
  qkv_tile(a.rows, a.N, QF_BM, QF_BN, tm, tn);
  if (tm * QF_BM >= a.rows) return;
  const int m0 = tm * QF_BM, n0 = tn * QF_BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wave & 1, wn = wave >> 1;
  const float* X = static_cast<const float*>(a.x);
  const float* Wt = static_cast<const float*>(a.w);
  const float* const bias = static_cast<const float*>(a.bias);
  float4 bq[2];  // the lane's bias, loaded before the contraction
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 32 * wn + 16 * j + 4 * g;
    bq[j] = (bias != nullptr && n < a.N) ? *reinterpret_cast<const float4*>(bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  f32x4 acc[2][2];  // [n subtile][m subtile]: y^T tiles
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.K; k0 += QF_BK) {
    // 64 rows x 8 float4 of each operand: 2 of each per thread
    float4 xa[2], xb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u, r = idx >> 3, c4 = idx & 7, k = k0 + 4 * c4;
      const bool kin = k < a.K;
      xa[u] = (m0 + r < a.rows && kin) ? *reinterpret_cast<const float4*>(X + (size_t)(m0 + r) * a.K + k)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
      xb[u] = (n0 + r < a.N && kin) ? *reinterpret_cast<const float4*>(Wt + (size_t)(n0 + r) * a.K + k)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();  // the previous step's reads are done
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u, r = idx >> 3, c4 = idx & 7;
      *reinterpret_cast<float4*>(As + r * QF_LD + 4 * c4) = xa[u];
      *reinterpret_cast<float4*>(Bs + r * QF_LD + 4 * c4) = xb[u];
    }
    __syncthreads();
    // k step s: lane (g, c16) feeds W[n][k0 + 4s + g] and x[m][k0 + 4s + g]
#pragma unroll
    for (int s4 = 0; s4 < QF_BK / 4; ++s4) {
      float av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = As[(32 * wm + 16 * i + c16) * QF_LD + 4 * s4 + g];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = Bs[(32 * wn + 16 * j + c16) * QF_LD + 4 * s4 + g];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[j][i] = mfma_f32(bv[j], av[i], acc[j][i]);
    }
  }
  float* const Y = static_cast<float*>(a.y);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 32 * wn + 16 * j + 4 * g;
    if (n >= a.N) continue;
    const float4 b4 = bq[j];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = m0 + 32 * wm + 16 * i + c16;
      if (m >= a.rows) continue;
      const f32x4 v = acc[j][i];
      *reinterpret_cast<float4*>(Y + (size_t)m * a.N + n) = make_float4(v[0] + b4.x, v[1] + b4.y, v[2] + b4.z, v[3] + b4.w);
    }
  }
}

}  // namespace nys
