// Backward pass: gradients of sum(out * dout) with respect to q, k, v and
// the convolution weights, for the Nystrom path.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), sections 2.2 -
// 2.6 (the forward that is differentiated: d^-1/4 scales, segment means,
// F = softmax(Qs Kt^T), A = softmax(Qt Kt^T), B = softmax(Qt Ks^T + mask),
// the iterative inverse Z from Z_0 = A^T / c, out = F (Z (B V)) + conv(V)),
// and its training use (gradient checkpointing, the Trainer).  The
// intermediates are recomputed (landmarks, A, Z, B V, W and B's row
// normalisers come from a forward pass without the output), then, per head
// (head size d = 32 or 64 with up to 256 landmarks, d = 128 with up to 64;
// float32 accumulation throughout; above 64 landmarks at d = 64 the token
// pass is k_bwd_tok3, above 128 landmarks the key pass takes the landmarks
// in two halves, and above 64 landmarks the per-head products run as a
// launch chain over all heads, k_bwd_chain):
//
//   k_bwd_dvconv  dv_conv = conv^T(dout) (the forward convolution with the
//               taps reversed, on the matrix cores);
//   k_bwd_conv  partial sums of dconv_w;
//   k_bwd_tok   per token: F, dF = dout W^T, D_t = sum_j F dF,
//               dS = F (dF - D_t), dQs = dS Kt; per token chunk partial
//               sums of dW = F^T dout and dKt = dS^T Qs (k_bwd_tok2 on the
//               bf16 matrix cores where d <= 64 and m d <= 64 * 64;
//               k_bwd_tok3, eight waves per token group with Kt and W in
//               LDS, at d = 64 above 64 landmarks);
//   k_bwd_mm1   per head: dW, dZ = dW BV^T, dBV = Z^T dW, the iteration run
//               backwards (Z_k, X_k, X_k^2 and P_k = 13I - 15X + 7X^2 - X^3
//               recomputed in float32 and kept), dA, and the part dc of the
//               gradient that flows through the initial scale c (above
//               64 landmarks the same products as the k_bwd_chain launches,
//               with k_bwd_chain_init / _stats / _sum / _post / _dc);
//   k_bwd_mm2   c's share of dA (through the maximum column sum: to the
//               arg-max column, of this head for init option 1, of the one
//               head holding the maximum over all heads for option 0; the
//               row-sum factor's share is constant along rows and vanishes
//               in the softmax), dS_A = A (dA - rowsum(dA A)),
//               dQt_A = dS_A Kt, dKt += dS_A^T Qt, D_i = dBV_i . BV_i;
//   k_bwd_key   per key: B from the stored normalisers, dB = dBV V^T,
//               dS_B = B (dB - D_i), dv = B^T dBV + dv_conv,
//               dk = d^-1/4 (dS_B^T Qt + dKt[segment] / L); per key chunk
//               partial sums of dQt_B = dS_B Ks (k_bwd_key2 on the bf16
//               matrix cores for the shapes of k_bwd_tok2);
//   k_bwd_qt    dQt = dQt_A + sum of the dQt_B partials;
//   k_bwd_q     dq = d^-1/4 (dQs + dQt[segment] / L);
//   k_bwd_wsum  dconv_w = sum of its partials.
// The per-head products and the token / key passes above 64 x 64 are
// float32 matrix-core products (mm16) over operands in LDS; k_bwd_tok2 and
// k_bwd_key2 use split-bf16 products (hi*hi + hi*lo + lo*hi, relative error
// about 2^-16; exact bf16 inputs skip their lo plane), as do the conv
// kernels.  Reductions run in a fixed order, so results are reproducible.
#pragma once

#include "common.hpp"
#include "k_conv.hpp"

namespace nys {

// C (16 x 16) += sum_k A(i, k) B(k, j) over k < K, with A(i, k) at
// a[i * ai + k * ak] and B(k, j) at b[k * bk + j * bj]: in step s lane
// (c16, g) feeds A(c16, 4s + g) and B(4s + g, c16); C(4g + r, c16) ends in
// element r.
// The k steps alternate between four accumulators (summed at the end, in a
// fixed order), so consecutive matrix-core operations do not wait on each
// other's results.
template <int K>
__device__ __forceinline__ f32x4 mm16(const float* a, int ai, int ak, const float* b, int bk, int bj, f32x4 c) {
  constexpr int NS = K / 4, NA = NS % 4 == 0 ? 4 : (NS % 2 == 0 ? 2 : 1);
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const float* pa = a + c16 * ai + g * ak;
  const float* pb = b + g * bk + c16 * bj;
  f32x4 acc[NA];
  acc[0] = c;
#pragma unroll
  for (int i = 1; i < NA; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) acc[s % NA] = mfma_f32(pa[4 * s * ak], pb[4 * s * bk], acc[s % NA]);
#pragma unroll
  for (int i = 1; i < NA; ++i) acc[0] += acc[i];
  return acc[0];
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const uint8_t* key_mask;  // [B][n] or null
  const float* conv_w;      // [H][conv_k] or null
  int conv_k;
  const float* qt;          // [BH][M][d] (carry d^-1/4)
  const float* kt;
  const float* A;           // [BH][M][M]
  const float* BV;          // [BH][M][d]
  const float* W;           // [BH][M][d]
  const float* lse;         // [BH][M], log2 units
  const float* cscale;      // [BH]
  float* dqf;               // [BH][n][d]: dQs through F
  float* pw;                // [BH][nct][M][d]: partial dW
  float* pk;                // [BH][nct][M][d]: partial dKt through F
  float* pq;                // [BH][nck][M][d]: partial dQt through B
  float* mm;                // [BH][mm_mats][M][M]: pseudo-inverse backward scratch
  float* dW;                // [BH][M][d]
  float* dBV;               // [BH][M][d]
  float* dQt;               // [BH][M][d]: dQt through A, then the total
  float* dKt;               // [BH][M][d]: total
  float* Dv;                // [BH][M]: dBV_i . BV_i
  float* dc;                // [BH]: gradient reaching c
  float* cmax;              // [BH]: maximum column sum of A
  int* cmaxj;               // [BH]: its column
  float* rmax;              // [BH]: maximum row sum of A
  float* dvc;               // [BH][n][d]: conv part of dv, or null
  float* dvk;               // [2][BH][n][d]: the key pass's first-half dv, dk (above 128 landmarks)
  float* pconv;             // [BH][ncv][conv_k]
  void* dq;
  void* dk;
  void* dv;
  float* dconv_w;           // [H][conv_k] or null
  int n, H, BH, mr, L, nct, nck, ncv, n_iter, init_option;
  float s4;                 // d^-1/4
};

// Kernels are templated on the head size D (32, 64 or 128); [.][D] float
// tiles in LDS have row stride D + 4.
constexpr int BWD_CT = 256;      // tokens per k_bwd_tok workgroup
constexpr int BWD_CK = 256;      // keys per k_bwd_key workgroup
constexpr int BWD_GK = 32;       // keys per step of k_bwd_key
constexpr int BWD_CV = 128;      // tokens per k_bwd_conv workgroup
constexpr int BWD_T3_CT = 512;   // tokens per k_bwd_tok3 workgroup
constexpr int BWD_CK2 = 512;     // keys per k_bwd_key workgroup above 128 landmarks
// the four-wave token pass for head size 64 above 64 landmarks
__host__ __device__ constexpr bool bwd_tok3(int M, int D) { return D == 64 && M > 64; }

template <int M>
constexpr int bwd_tok_waves() {
  return M <= 64 ? 4 : 2;
}
// matrices of the pseudo-inverse backward per head: Z_0 .. Z_n, then X_k,
// X_k^2, P_k for k < n, then G, Gn, dP, dX, T, dA
__host__ __device__ constexpr int bwd_mm_mats(int n_iter) { return 4 * n_iter + 1 + 6; }

template <typename IO>
__device__ __forceinline__ float io_get(const IO* p) {
  if constexpr (sizeof(IO) == 4)
    return *reinterpret_cast<const float*>(p);
  else
    return bf16u_to_f32(*reinterpret_cast<const u16*>(p));
}
template <typename IO>
__device__ __forceinline__ void io_put(IO* p, float x) {
  if constexpr (sizeof(IO) == 4)
    *reinterpret_cast<float*>(p) = x;
  else
    *reinterpret_cast<u16*>(p) = f32_to_bf16u(x);
}
// Four consecutive elements (16-byte aligned for float32, 8-byte for bf16).
template <typename IO>
__device__ __forceinline__ void io_put4(IO* p, const f32x4 x) {
  if constexpr (sizeof(IO) == 4)
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}

// ---------------------------------------------------------------------------
template <int M, int D>
struct BwdTokLayout {
  static constexpr int NW = bwd_tok_waves<M>(), GT = 16 * NW, LDF = M + 4, LD = D + 4;
  // Above 128 landmarks the key landmarks stay in L2, and at d = 64 the pass
  // is split by channels: workgroup z of a token chunk accumulates dW, dKt
  // and writes dQs for channels [z DC, (z + 1) DC) only (each half forms the
  // whole S, dF and softmax of its tokens; the halves share nothing).
  static constexpr bool KT_LDS = M <= 128;
  // S and dF through LDS rather than whole rows in registers
  static constexpr bool S_LDS = M > 128;
  static constexpr int SPLIT = (M > 128 && D > 32) ? 2 : 1;
  static constexpr int DC = D / SPLIT, LDC = DC + 4;
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_Q = OFF_KT + (KT_LDS ? M * LD : 0);
  static constexpr int OFF_DO = OFF_Q + GT * LD;
  static constexpr int OFF_F = OFF_DO + GT * LD;
  static constexpr int OFF_DS = OFF_F + GT * LDF;
  // the dW / dKt accumulators: in registers (each wave owns fixed tiles) up
  // to 64 landmarks, in LDS above
  static constexpr bool ACC_REG = M <= 64;
  static constexpr int OFF_AW = OFF_DS + GT * LDF;
  static constexpr int OFF_AK = OFF_AW + (ACC_REG ? 0 : M * LDC);
  static constexpr int OFF_W = OFF_AK + (ACC_REG ? 0 : M * LDC);
  // W is staged too where it fits (otherwise read from L2)
  static constexpr bool W_LDS = 4 * (OFF_W + M * LD) <= 160 * 1024;
  static constexpr int FLOATS = OFF_W + (W_LDS ? M * LD : 0);
  static constexpr int BYTES = 4 * FLOATS;
  static_assert(BYTES <= 160 * 1024, "k_bwd_tok LDS");
  static_assert(!ACC_REG || SPLIT == 1, "register accumulators cover every channel");
};

// grid (nct, BH, Ly::SPLIT), block 64 NW.
template <typename IO, int M, int D>
__global__ __launch_bounds__(64 * bwd_tok_waves<M>()) void k_bwd_tok(BwdArgs a) {
  extern __shared__ __align__(16) float bw_lds[];
  using Ly = BwdTokLayout<M, D>;
  constexpr int NW = Ly::NW, GT = Ly::GT, LDF = Ly::LDF, LD = Ly::LD, TM = M / 16, CT = D / 16;
  constexpr int DC = Ly::DC, LDC = Ly::LDC, CTC = DC / 16;  // this workgroup's channels
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int ct0 = blockIdx.z * CTC;  // first channel tile of this workgroup
  const int t0 = chunk * BWD_CT, t1 = min(a.n, t0 + BWD_CT);
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const float* Wg = a.W + (size_t)bh * M * D;
  const float* const Kt = Ly::KT_LDS ? bw_lds + Ly::OFF_KT : a.kt + (size_t)bh * M * D;
  constexpr int KLD = Ly::KT_LDS ? LD : D;
  float* const Qg = bw_lds + Ly::OFF_Q;
  float* const DOg = bw_lds + Ly::OFF_DO;
  float* const Fg = bw_lds + Ly::OFF_F;
  float* const DSg = bw_lds + Ly::OFF_DS;
  float* const AW = bw_lds + Ly::OFF_AW;
  float* const AK = bw_lds + Ly::OFF_AK;
  float* const Wl = bw_lds + Ly::OFF_W;
  const float* const Wsrc = Ly::W_LDS ? Wl : Wg;
  constexpr int WLD = Ly::W_LDS ? LD : D;
  for (int i = threadIdx.x; i < M * D; i += 64 * NW) {
    if constexpr (Ly::KT_LDS) bw_lds[Ly::OFF_KT + (i / D) * LD + i % D] = a.kt[(size_t)bh * M * D + i];
    if constexpr (Ly::W_LDS) Wl[(i / D) * LD + i % D] = Wg[i];
  }
  if constexpr (!Ly::ACC_REG) {
    for (int i = threadIdx.x; i < M * DC; i += 64 * NW) {
      AW[(i / DC) * LDC + i % DC] = 0.f;
      AK[(i / DC) * LDC + i % DC] = 0.f;
    }
  }
  constexpr int NACC = Ly::ACC_REG ? 2 * TM * CT / NW : 1;
  static_assert(!Ly::ACC_REG || (2 * TM * CT) % NW == 0, "every wave owns the same number of tiles");
  f32x4 racc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) racc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int gs = t0; gs < t1; gs += GT) {
    // ---- phase A: the wave's 16 tokens (4 lanes per token, D / 4 channels each)
    const int tw = gs + 16 * wave;
    {
      const int r = lane >> 2, c0 = (D / 4) * (lane & 3), tok = tw + r;
      float* qd = Qg + (16 * wave + r) * LD + c0;
      float* od = DOg + (16 * wave + r) * LD + c0;
#pragma unroll
      for (int h = 0; h < D / 32; ++h) {
        float xq[8], xo[8];
        if (tok < t1) {
          IOTraits<IO>::load8(Q + (size_t)tok * D + c0 + 8 * h, xq);
          IOTraits<IO>::load8(DO + (size_t)tok * D + c0 + 8 * h, xo);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[e] = xo[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qd[8 * h + e] = xq[e] * a.s4;
          od[8 * h + e] = xo[e];
        }
      }
    }
    // S = Qs Kt^T and dF = dout W^T: C(token 4g + r, landmark 16 jt + c16)
    if constexpr (Ly::S_LDS) {
      // above 128 landmarks S and dF go to LDS one tile at a time (whole
      // rows of both stay out of the registers), then the row softmax runs
      // over the wave's 16 rows there, four lanes per row
#pragma unroll 1
      for (int jt = 0; jt < TM; ++jt) {
        f32x4 f = mm16<D>(Qg + 16 * wave * LD, LD, 1, Kt + 16 * jt * KLD, 1, KLD, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 df = mm16<D>(DOg + 16 * wave * LD, LD, 1, Wsrc + 16 * jt * WLD, 1, WLD, f32x4{0.f, 0.f, 0.f, 0.f});
        if (16 * jt + c16 >= a.mr) f = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * wave + 4 * g + r;
          Fg[row * LDF + 16 * jt + c16] = f[r];
          DSg[row * LDF + 16 * jt + c16] = df[r];
        }
      }
      __syncthreads();
      {
        const int row = 16 * wave + (lane >> 2), q4 = lane & 3;
        float* const fr = Fg + row * LDF;
        float* const dr = DSg + row * LDF;
        float mx = -INFINITY;
        for (int c = q4; c < M; c += 4) mx = fmaxf(mx, fr[c]);
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        float s = 0.f;
        for (int c = q4; c < M; c += 4) {
          const float e = __expf(fr[c] - mx);
          fr[c] = e;
          s += e;
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        const float inv = 1.0f / s;
        float dt = 0.f;
        for (int c = q4; c < M; c += 4) {
          const float fv = fr[c] * inv;
          fr[c] = fv;
          dt += fv * dr[c];
        }
        dt += __shfl_xor(dt, 1);
        dt += __shfl_xor(dt, 2);
        for (int c = q4; c < M; c += 4) dr[c] = fr[c] * (dr[c] - dt);
      }
      __syncthreads();
    } else {
      f32x4 f[TM], df[TM];
#pragma unroll
      for (int jt = 0; jt < TM; ++jt) {
        f[jt] = mm16<D>(Qg + 16 * wave * LD, LD, 1, Kt + 16 * jt * KLD, 1, KLD, f32x4{0.f, 0.f, 0.f, 0.f});
        df[jt] = mm16<D>(DOg + 16 * wave * LD, LD, 1, Wsrc + 16 * jt * WLD, 1, WLD, f32x4{0.f, 0.f, 0.f, 0.f});
        if (16 * jt + c16 >= a.mr) f[jt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) mx = fmaxf(mx, f[jt][r]);
        mx = max16(mx);
        float s = 0.f;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) {
          f[jt][r] = __expf(f[jt][r] - mx);
          s += f[jt][r];
        }
        const float inv = 1.0f / sum16(s);
        float dt = 0.f;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) {
          f[jt][r] *= inv;
          dt += f[jt][r] * df[jt][r];
        }
        dt = sum16(dt);
        const int row = 16 * wave + 4 * g + r;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) {
          Fg[row * LDF + 16 * jt + c16] = f[jt][r];
          DSg[row * LDF + 16 * jt + c16] = f[jt][r] * (df[jt][r] - dt);
        }
      }
    }
    // dQs = dS Kt (16 tokens x this workgroup's channels), the wave's own rows
#pragma unroll
    for (int cc = 0; cc < CTC; ++cc) {
      const int ct = ct0 + cc;
      const f32x4 c = mm16<M>(DSg + 16 * wave * LDF, LDF, 1, Kt + 16 * ct, KLD, 1, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tw + 4 * g + r;
        if (tok < t1) a.dqf[((size_t)bh * a.n + tok) * D + 16 * ct + c16] = c[r];
      }
    }
    __syncthreads();
    // ---- phase B: dW += F^T dout and dKt += dS^T Qs over the group's tokens;
    // tile ti = (landmark tile jt, channel tile ct), the dKt tiles after the dW tiles
    if constexpr (Ly::ACC_REG) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        const int ti = wave + NW * j;
        const bool isk = ti >= TM * CT;
        const int tt = ti % (TM * CT), jt = tt / CT, ct = tt % CT;
        const float* A0 = (isk ? DSg : Fg) + 16 * jt;
        const float* B0 = (isk ? Qg : DOg) + 16 * ct;
        racc[j] = mm16<GT>(A0, 1, LDF, B0, LD, 1, racc[j]);
      }
    } else {
      for (int ti = wave; ti < 2 * TM * CTC; ti += NW) {
        const bool isk = ti >= TM * CTC;
        const int tt = ti % (TM * CTC), jt = tt / CTC, cc = tt % CTC;
        const float* A0 = (isk ? DSg : Fg) + 16 * jt;
        const float* B0 = (isk ? Qg : DOg) + 16 * (ct0 + cc);
        const f32x4 c = mm16<GT>(A0, 1, LDF, B0, LD, 1, f32x4{0.f, 0.f, 0.f, 0.f});
        float* acc = (isk ? AK : AW) + (16 * jt + 4 * g) * LDC + 16 * cc + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r * LDC] += c[r];
      }
    }
    __syncthreads();
  }
  float* const pw = a.pw + ((size_t)bh * a.nct + chunk) * M * D;
  float* const pk = a.pk + ((size_t)bh * a.nct + chunk) * M * D;
  if constexpr (Ly::ACC_REG) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      const int ti = wave + NW * j;
      const bool isk = ti >= TM * CT;
      const int tt = ti % (TM * CT), jt = tt / CT, ct = tt % CT;
      float* const dst = isk ? pk : pw;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * jt + 4 * g + r) * D + 16 * ct + c16] = racc[j][r];
    }
  } else {
    for (int i = threadIdx.x; i < M * DC; i += 64 * NW) {
      const int r = i / DC, c = i % DC;
      pw[(size_t)r * D + 16 * ct0 + c] = AW[r * LDC + c];
      pk[(size_t)r * D + 16 * ct0 + c] = AK[r * LDC + c];
    }
  }
}

// ---------------------------------------------------------------------------
// Token pass for head size 64 above 64 landmarks: eight waves share each
// 32-token group, Kt (and W where it fits) stay in LDS for the whole chunk,
// and every wave holds its share of the dW / dKt tiles in registers:
//   S = Qs Kt^T and dF = dout W^T tile by tile into LDS (the 2 x M/16 tile
//   pairs dealt over the waves), the row softmax there (sixteen lanes per
//   row), dS = F (dF - D_t); dQs = dS Kt (eight 16 x 16 tiles, one per
//   wave); dW += F^T dout and dKt += dS^T Qs over the group's tokens
//   (2 M/16 x 4 tiles, M/16 per wave).
// Float32 matrix-core products (mm16) over float32 LDS operands, except at
// bf16 I/O: there S, dF, dW and dKt run on v_mfma_f32_16x16x32_bf16 with
// dout and q as exact bf16 operands (q staged unscaled; S and the dKt
// partials take the d^-1/4 instead) and Kt, W, F, dS split hi + lo (two
// products per 32-element contraction block; relative error about 2^-16).
// Up to 192 landmarks dQs does too (three products per block, hi hi, hi lo,
// lo hi): a wave's dQs tile has the same channel tile all through the
// chunk, so its Kt fragments are split once into registers.
template <int M>
struct BwdTok3Layout {
  static constexpr int D = 64, NW = 8, GT = 32, LDF = M + 4, LD = D + 4;
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_Q = OFF_KT + M * LD;
  static constexpr int OFF_DO = OFF_Q + GT * LD;
  static constexpr int OFF_F = OFF_DO + GT * LD;
  static constexpr int OFF_DS = OFF_F + GT * LDF;
  static constexpr int OFF_W = OFF_DS + GT * LDF;
  static constexpr bool W_LDS = 4 * (OFF_W + M * LD) <= 160 * 1024;
  static constexpr int FLOATS = OFF_W + (W_LDS ? M * LD : 0);
  static constexpr int BYTES = 4 * FLOATS;
  static_assert(BYTES <= 160 * 1024, "k_bwd_tok3 LDS");
};

// grid (nct, BH), block 64 BwdTok3Layout::NW.
template <typename IO, int M>
__global__ __launch_bounds__(64 * BwdTok3Layout<M>::NW) void k_bwd_tok3(BwdArgs a) {
  extern __shared__ __align__(16) float bw_lds[];
  using Ly = BwdTok3Layout<M>;
  constexpr int D = 64, NW = Ly::NW, GT = Ly::GT, LDF = Ly::LDF, LD = Ly::LD, TM = M / 16, CT = D / 16;
  constexpr int NACC = 2 * TM * CT / NW;
  constexpr int NTH = 64 * NW, LPR = NTH / GT;  // threads; lanes per row in the softmax
  static_assert((2 * TM * CT) % NW == 0 && M % 16 == 0, "every wave owns the same number of tiles");
  static_assert(NTH >= 8 * GT && LPR <= 64 && (LPR & (LPR - 1)) == 0, "staging and softmax lane layout");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int t0 = chunk * BWD_T3_CT, t1 = min(a.n, t0 + BWD_T3_CT);
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const float* const Wg = a.W + (size_t)bh * M * D;
  const float* const Ktg = a.kt + (size_t)bh * M * D;
  float* const Kt = bw_lds + Ly::OFF_KT;
  float* const Qg = bw_lds + Ly::OFF_Q;
  float* const DOg = bw_lds + Ly::OFF_DO;
  float* const Fg = bw_lds + Ly::OFF_F;
  float* const DSg = bw_lds + Ly::OFF_DS;
  float* const Wl = bw_lds + Ly::OFF_W;
  const float* const Wsrc = Ly::W_LDS ? Wl : Wg;
  constexpr int WLD = Ly::W_LDS ? LD : D;
  constexpr bool BF = sizeof(IO) == 2;  // dW / dKt on the bf16 matrix cores
  const float qs = BF ? 1.f : a.s4;     // the scale staged with q
  for (int i = tid; i < M * D / 4; i += NTH) {
    const int r = i / (D / 4), c = 4 * (i % (D / 4));
    *reinterpret_cast<float4*>(Kt + r * LD + c) = *reinterpret_cast<const float4*>(Ktg + (size_t)r * D + c);
    if constexpr (Ly::W_LDS)
      *reinterpret_cast<float4*>(Wl + r * LD + c) = *reinterpret_cast<const float4*>(Wg + (size_t)r * D + c);
  }
  f32x4 racc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) racc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // dQs on bf16 products: one tile per wave (token tile wave / CT, channel
  // tile wave % CT), B(landmark 32 kb + 8g + e, channel c16) fragments of Kt
  constexpr bool BFQ = BF && M <= 192 && M % 32 == 0 && 2 * CT == NW;
  constexpr int NKB = BFQ ? M / 32 : 1;
  Frag2 fk[NKB];
  if constexpr (BFQ) {
    __syncthreads();  // Kt staged
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float xk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xk[e] = Kt[(32 * kb + 8 * g + e) * LD + 16 * (wave % CT) + c16];
      fk[kb] = split8(xk);
    }
  }
  for (int gs = t0; gs < t1; gs += GT) {
    // q (scaled) and dout rows of the group: eight lanes per token, eight channels each
    if (tid < 8 * GT) {
      const int r = tid >> 3, c0 = 8 * (tid & 7), tok = gs + r;
      float xq[8], xo[8];
      if (tok < t1) {
        IOTraits<IO>::load8(Q + (size_t)tok * D + c0, xq);
        IOTraits<IO>::load8(DO + (size_t)tok * D + c0, xo);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xq[e] = xo[e] = 0.f;
      }
      float* const qd = Qg + r * LD + c0;
      float* const od = DOg + r * LD + c0;
      *reinterpret_cast<float4*>(qd) = make_float4(xq[0] * qs, xq[1] * qs, xq[2] * qs, xq[3] * qs);
      *reinterpret_cast<float4*>(qd + 4) = make_float4(xq[4] * qs, xq[5] * qs, xq[6] * qs, xq[7] * qs);
      *reinterpret_cast<float4*>(od) = make_float4(xo[0], xo[1], xo[2], xo[3]);
      *reinterpret_cast<float4*>(od + 4) = make_float4(xo[4], xo[5], xo[6], xo[7]);
    }
    __syncthreads();  // rows staged (and, the first time, Kt / W)
    // S and dF tile pairs p = (token tile p % 2, landmark tile p / 2): C(token 4g + r, landmark c16)
    // at bf16 I/O a wave's token tile is p & 1 = wave & 1 for all its pairs
    // (NW even): its q and dout fragments (token c16, channels 32 kb + 8g + e)
    // are formed once
    static_assert(NW % 2 == 0, "a fixed token tile per wave");
    bf16x8 aq[D / 32], ado[D / 32];
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const float* const qr = Qg + (16 * (wave & 1) + c16) * LD + 32 * kb + 8 * g;
        const float* const dr = DOg + (16 * (wave & 1) + c16) * LD + 32 * kb + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          aq[kb][e] = (__bf16)qr[e];
          ado[kb][e] = (__bf16)dr[e];
        }
      }
    }
    for (int p = wave; p < 2 * TM; p += NW) {
      const int tt = p & 1, jt = p >> 1;
      f32x4 f, df;
      if constexpr (BF) {
        f = df = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
          const Frag2 bk = split8(Kt + (16 * jt + c16) * LD + 32 * kb + 8 * g);
          const Frag2 bw = split8(Wsrc + (16 * jt + c16) * WLD + 32 * kb + 8 * g);
          f = mfma(aq[kb], bk.hi, f);
          f = mfma(aq[kb], bk.lo, f);
          df = mfma(ado[kb], bw.hi, df);
          df = mfma(ado[kb], bw.lo, df);
        }
        f *= a.s4;
      } else {
        f = mm16<D>(Qg + 16 * tt * LD, LD, 1, Kt + 16 * jt * LD, 1, LD, f32x4{0.f, 0.f, 0.f, 0.f});
        df = mm16<D>(DOg + 16 * tt * LD, LD, 1, Wsrc + 16 * jt * WLD, 1, WLD, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      if (16 * jt + c16 >= a.mr) f = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * tt + 4 * g + r;
        Fg[row * LDF + 16 * jt + c16] = f[r];
        DSg[row * LDF + 16 * jt + c16] = df[r];
      }
    }
    __syncthreads();
    // row softmax and dS, LPR lanes per row
    {
      const int row = tid / LPR, q = tid % LPR;
      float* const fr = Fg + row * LDF;
      float* const dr = DSg + row * LDF;
      float mx = -INFINITY;
      for (int c = q; c < M; c += LPR) mx = fmaxf(mx, fr[c]);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      float s = 0.f;
      for (int c = q; c < M; c += LPR) {
        const float e = __expf(fr[c] - mx);
        fr[c] = e;
        s += e;
      }
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
      const float inv = 1.0f / s;
      float dt = 0.f;
      for (int c = q; c < M; c += LPR) {
        const float fv = fr[c] * inv;
        fr[c] = fv;
        dt += fv * dr[c];
      }
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) dt += __shfl_xor(dt, o);
      for (int c = q; c < M; c += LPR) dr[c] = fr[c] * (dr[c] - dt);
    }
    __syncthreads();
    // dQs = dS Kt: tiles (token tile, channel tile) dealt over the waves
    for (int p = wave; p < 2 * CT; p += NW) {
      const int tt = p / CT, ct = p % CT;
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BFQ) {
        // A(token c16, landmark 32 kb + 8g + e)
        const float* const ar = DSg + (16 * tt + c16) * LDF + 8 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) c = mma<3>(split8(ar + 32 * kb), fk[kb], c);
      } else {
        c = mm16<M>(DSg + 16 * tt * LDF, LDF, 1, Kt + 16 * ct, LD, 1, c);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = gs + 16 * tt + 4 * g + r;
        if (tok < t1) a.dqf[((size_t)bh * a.n + tok) * D + 16 * ct + c16] = c[r];
      }
    }
    // dW += F^T dout and dKt += dS^T Qs; tile ti = (landmark tile, channel tile), the dKt tiles after the dW tiles
    if constexpr (BF) {
      // a wave's channel tile is the same for all of its tiles (NW % CT == 0):
      // its dout and q fragments (token 8g + e, channel c16) are formed once
      static_assert(NW % CT == 0 && GT == 32, "one 16 x 16 x 32 product per tile");
      const int ctw = wave % CT;
      bf16x8 bdo, bq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bdo[e] = (__bf16)DOg[(8 * g + e) * LD + 16 * ctw + c16];
        bq[e] = (__bf16)Qg[(8 * g + e) * LD + 16 * ctw + c16];
      }
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        const int ti = wave + NW * j;
        const bool isk = ti >= TM * CT;
        const int jt = (ti % (TM * CT)) / CT;
        const float* const X = (isk ? DSg : Fg) + 16 * jt + c16;
        float xa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[e] = X[(8 * g + e) * LDF];
        const Frag2 fa = split8(xa);
        const bf16x8 b = isk ? bq : bdo;
        racc[j] = mfma(fa.hi, b, racc[j]);
        racc[j] = mfma(fa.lo, b, racc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        const int ti = wave + NW * j;
        const bool isk = ti >= TM * CT;
        const int tt = ti % (TM * CT), jt = tt / CT, ct = tt % CT;
        const float* A0 = (isk ? DSg : Fg) + 16 * jt;
        const float* B0 = (isk ? Qg : DOg) + 16 * ct;
        racc[j] = mm16<GT>(A0, 1, LDF, B0, LD, 1, racc[j]);
      }
    }
    __syncthreads();  // the group's rows free
  }
  float* const pw = a.pw + ((size_t)bh * a.nct + chunk) * M * D;
  float* const pk = a.pk + ((size_t)bh * a.nct + chunk) * M * D;
#pragma unroll
  for (int j = 0; j < NACC; ++j) {
    const int ti = wave + NW * j;
    const bool isk = ti >= TM * CT;
    const int tt = ti % (TM * CT), jt = tt / CT, ct = tt % CT;
    float* const dst = isk ? pk : pw;
    const float sc = BF && isk ? a.s4 : 1.f;  // q was staged unscaled
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(size_t)(16 * jt + 4 * g + r) * D + 16 * ct + c16] = sc * racc[j][r];
  }
}

// ---------------------------------------------------------------------------
// Token pass on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16), for
// D <= 64 and M * D <= 64 * 64 (the LDS tiles and register accumulators
// grow with both).  Float32 operands are split hi + lo (products hi*hi +
// hi*lo + lo*hi, relative error about 2^-16); q and dout rows of bf16 I/O
// are exact bf16, so their products take two passes.  Each wave works alone
// on 32-token steps (steps wave, wave + 4, ... of the workgroup's chunk):
//   S = q Kt^T (then * d^-1/4) and dF = dout W^T for its two 16-token
//   tiles (q, dout rows staged in the wave's own LDS area; Kt, W staged
//   once per workgroup), the row softmax, dS = F (dF - D_t);
//   dW += F^T dout and dKt += dS^T q over the 32 tokens: the contraction
//   runs over tokens in the paired k order, which is exactly what the two
//   tiles' C registers hold, so F and dS enter as A operands straight from
//   registers and dout, q as B operands by transposed LDS reads;
//   dQs = dS Kt: dS^T goes to the wave's LDS tile, read back transposed;
//   the product is formed as dQs^T, so a lane stores 4 channels of a token.
// dW and dKt stay in registers over all of a wave's steps; at the end the
// four waves' sums are added in wave order and written as the chunk's
// partials.  No workgroup barrier inside the token loop.
constexpr int BWD_T2_CT = 1024;  // tokens per workgroup

__host__ __device__ constexpr bool bwd_tok2(int M, int D) { return D <= 64 && M * D <= 64 * 64; }
// tokens per token-pass workgroup (the chunk of one dW / dKt partial)
__host__ __device__ constexpr int bwd_tok_chunk(int M, int D) {
  return bwd_tok2(M, D) ? BWD_T2_CT : (bwd_tok3(M, D) ? BWD_T3_CT : BWD_CT);
}
// keys per key-pass workgroup (the chunk of one dQt partial)
constexpr int BWD_K2_CK = 1024;  // k_bwd_key2
__host__ __device__ constexpr int bwd_key_chunk(int M, int D) {
  return bwd_tok2(M, D) ? BWD_K2_CK : (M > 128 ? BWD_CK2 : BWD_CK);
}

template <typename IO, int M, int D>
struct BwdTok2Layout {
  static constexpr int NSQ = sizeof(IO) == 2 ? 1 : 2;  // bf16 planes of the staged q / dout rows
  static constexpr int KLD = D + 8;                    // element row stride of Kt, W, q, dout tiles
  static constexpr int SLD = 32 + 4;                   // element row stride of the dS^T tile
  // offsets in bf16 elements
  static constexpr int KT = 0;                    // Kt hi, lo planes [M][KLD]
  static constexpr int WT = KT + 2 * M * KLD;     // W hi, lo
  static constexpr int WAVE0 = WT + 2 * M * KLD;  // per-wave areas
  static constexpr int QW = 0;                    // q rows [32][KLD], NSQ planes
  static constexpr int DW = QW + NSQ * 32 * KLD;  // dout rows
  static constexpr int SW = DW + NSQ * 32 * KLD;  // dS^T hi, lo [M][SLD]
  static constexpr int PER_WAVE = SW + 2 * M * SLD;
  static constexpr int BYTES = 2 * (WAVE0 + 4 * PER_WAVE);
  static_assert(BYTES <= 160 * 1024, "k_bwd_tok2 LDS");
  static_assert(4 * M * D <= BYTES, "the epilogue sums [M][D] floats in LDS");
};

// N consecutive elements of one I/O row, held in registers between a global
// load and its LDS store (bf16: raw bits, stored as the exact hi plane;
// float32: split into hi and lo planes at the store).
template <typename IO, int N>
struct RowBuf;
template <int N>
struct RowBuf<u16, N> {
  uint4 v[N / 8];
  __device__ __forceinline__ void load(const u16* p, bool ok) {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) v[i] = ok ? *reinterpret_cast<const uint4*>(p + 8 * i) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(__bf16* hi, __bf16*) const {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) *reinterpret_cast<uint4*>(hi + 8 * i) = v[i];
  }
};
template <int N>
struct RowBuf<float, N> {
  float4 v[N / 4];
  __device__ __forceinline__ void load(const float* p, bool ok) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i)
      v[i] = ok ? *reinterpret_cast<const float4*>(p + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ void store(__bf16* hi, __bf16* lo) const {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const float x[8] = {v[2 * i].x, v[2 * i].y, v[2 * i].z, v[2 * i].w,
                          v[2 * i + 1].x, v[2 * i + 1].y, v[2 * i + 1].z, v[2 * i + 1].w};
      const Frag2 f = split8(x);
      *reinterpret_cast<bf16x8*>(hi + 8 * i) = f.hi;
      *reinterpret_cast<bf16x8*>(lo + 8 * i) = f.lo;
    }
  }
};

// B operand of rows k0 .. k0 + 3 and k1 .. k1 + 3 (element e < 4: row k0 + e,
// e >= 4: row k1 + e - 4) and column col0 + lane % 16 of a row-major bf16
// tile (row stride ld), by two transposed reads.
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* X, int ld, int k0, int k1, int col0) {
  const int c16 = threadIdx.x & 15;
  const int off = (c16 >> 2) * ld + col0 + 4 * (c16 & 3);
  return cat44(lds_read_tr(X + k0 * ld + off), lds_read_tr(X + k1 * ld + off));
}

// grid (ceil(n / BWD_T2_CT), BH), block 256, dynamic LDS BwdTok2Layout::BYTES.
template <typename IO, int M, int D>
__global__ __launch_bounds__(256) void k_bwd_tok2(BwdArgs a) {
  extern __shared__ __align__(16) __bf16 t2_lds[];
  using Ly = BwdTok2Layout<IO, M, D>;
  constexpr int NSQ = Ly::NSQ, KLD = Ly::KLD, SLD = Ly::SLD;
  constexpr int TM = M / 16, CT = D / 16, KD = D / 32, KM = M / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int t0 = chunk * BWD_T2_CT, t1 = min(a.n, t0 + BWD_T2_CT);
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  __bf16* const Kh = t2_lds + Ly::KT;
  __bf16* const Kl = Kh + M * KLD;
  __bf16* const Wh = t2_lds + Ly::WT;
  __bf16* const Wl = Wh + M * KLD;
  __bf16* const wb = t2_lds + Ly::WAVE0 + wave * Ly::PER_WAVE;
  __bf16* const Qp = wb + Ly::QW;  // plane p at Qp + p * 32 * KLD
  __bf16* const Dp = wb + Ly::DW;
  __bf16* const Sh = wb + Ly::SW;
  __bf16* const Sl = Sh + M * SLD;

  // Kt and W (float32 [M][D]) as bf16 hi / lo planes
  for (int i = threadIdx.x; i < M * D / 8; i += 256) {
    const int r = i / (D / 8), c = 8 * (i % (D / 8));
    float x[8];
    IOTraits<float>::load8(a.kt + ((size_t)bh * M + r) * D + c, x);
    const Frag2 fk = split8(x);
    *reinterpret_cast<bf16x8*>(Kh + r * KLD + c) = fk.hi;
    *reinterpret_cast<bf16x8*>(Kl + r * KLD + c) = fk.lo;
    IOTraits<float>::load8(a.W + ((size_t)bh * M + r) * D + c, x);
    const Frag2 fw = split8(x);
    *reinterpret_cast<bf16x8*>(Wh + r * KLD + c) = fw.hi;
    *reinterpret_cast<bf16x8*>(Wl + r * KLD + c) = fw.lo;
  }

  // staging lanes: token lane / 2 of the step, channels (lane % 2) D / 2 ..
  const int sr = lane >> 1, sc = (lane & 1) * (D / 2);
  const int nsteps = (t1 - t0 + 31) / 32;
  RowBuf<IO, D / 2> bq, bd;
  auto fetch = [&](int step) {
    const int tok = t0 + 32 * step + sr;
    const bool ok = tok < t1;
    const size_t o = (size_t)(ok ? tok : t0) * D + sc;
    bq.load(Q + o, ok);
    bd.load(DO + o, ok);
  };
  if (wave < nsteps) fetch(wave);
  f32x4 accW[TM][CT], accK[TM][CT];
#pragma unroll
  for (int jt = 0; jt < TM; ++jt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) accW[jt][ct] = accK[jt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // Kt, W staged

  for (int step = wave; step < nsteps; step += 4) {
    const int ts = t0 + 32 * step;
    // this step's rows into the wave's area (its reads of the last step are
    // done: a wave's LDS accesses complete in order), then the next fetch
    bq.store(Qp + sr * KLD + sc, Qp + 32 * KLD + sr * KLD + sc);
    bd.store(Dp + sr * KLD + sc, Dp + 32 * KLD + sr * KLD + sc);
    if (step + 4 < nsteps) fetch(step + 4);

    // S = q Kt^T and dF = dout W^T: C(token 16 rt + 4g + r, landmark 16 jt + c16)
    f32x4 s[2][TM], df[2][TM];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      Frag2 qa[KD], da[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        const int o = (16 * rt + c16) * KLD + 32 * ks + 8 * g;
        qa[ks].hi = *reinterpret_cast<const bf16x8*>(Qp + o);
        da[ks].hi = *reinterpret_cast<const bf16x8*>(Dp + o);
        if constexpr (NSQ == 2) {
          qa[ks].lo = *reinterpret_cast<const bf16x8*>(Qp + 32 * KLD + o);
          da[ks].lo = *reinterpret_cast<const bf16x8*>(Dp + 32 * KLD + o);
        }
      }
#pragma unroll
      for (int jt = 0; jt < TM; ++jt) {
        f32x4 cs = f32x4{0.f, 0.f, 0.f, 0.f}, cd = cs;
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          const int o = (16 * jt + c16) * KLD + 32 * ks + 8 * g;
          const bf16x8 kh = *reinterpret_cast<const bf16x8*>(Kh + o);
          const bf16x8 kl = *reinterpret_cast<const bf16x8*>(Kl + o);
          const bf16x8 wh = *reinterpret_cast<const bf16x8*>(Wh + o);
          const bf16x8 wl = *reinterpret_cast<const bf16x8*>(Wl + o);
          cs = mfma(qa[ks].hi, kh, cs);
          cs = mfma(qa[ks].hi, kl, cs);
          cd = mfma(da[ks].hi, wh, cd);
          cd = mfma(da[ks].hi, wl, cd);
          if constexpr (NSQ == 2) {
            cs = mfma(qa[ks].lo, kh, cs);
            cd = mfma(da[ks].lo, wh, cd);
          }
        }
        s[rt][jt] = cs * a.s4;
        df[rt][jt] = cd;
        if (16 * jt + c16 >= a.mr) s[rt][jt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
    // row softmax F and dS = F (dF - D_t), in place of s and df
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) mx = fmaxf(mx, s[rt][jt][r]);
        mx = max16(mx);
        float sum = 0.f;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) {
          s[rt][jt][r] = __expf(s[rt][jt][r] - mx);
          sum += s[rt][jt][r];
        }
        const float inv = 1.0f / sum16(sum);
        float dt = 0.f;
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) {
          s[rt][jt][r] *= inv;
          dt += s[rt][jt][r] * df[rt][jt][r];
        }
        dt = sum16(dt);
#pragma unroll
        for (int jt = 0; jt < TM; ++jt) df[rt][jt][r] = s[rt][jt][r] * (df[rt][jt][r] - dt);
      }
    // dW += F^T dout, dKt += dS^T q over the step's 32 tokens (paired k order)
#pragma unroll
    for (int jt = 0; jt < TM; ++jt) {
      const float fx[8] = {s[0][jt][0], s[0][jt][1], s[0][jt][2], s[0][jt][3],
                           s[1][jt][0], s[1][jt][1], s[1][jt][2], s[1][jt][3]};
      const float sx[8] = {df[0][jt][0], df[0][jt][1], df[0][jt][2], df[0][jt][3],
                           df[1][jt][0], df[1][jt][1], df[1][jt][2], df[1][jt][3]};
      const Frag2 fa = split8(fx), sa = split8(sx);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 dbh = tr_frag(Dp, KLD, 4 * g, 16 + 4 * g, 16 * ct);
        const bf16x8 qbh = tr_frag(Qp, KLD, 4 * g, 16 + 4 * g, 16 * ct);
        accW[jt][ct] = mfma(fa.hi, dbh, accW[jt][ct]);
        accW[jt][ct] = mfma(fa.lo, dbh, accW[jt][ct]);
        accK[jt][ct] = mfma(sa.hi, qbh, accK[jt][ct]);
        accK[jt][ct] = mfma(sa.lo, qbh, accK[jt][ct]);
        if constexpr (NSQ == 2) {
          accW[jt][ct] = mfma(fa.hi, tr_frag(Dp + 32 * KLD, KLD, 4 * g, 16 + 4 * g, 16 * ct), accW[jt][ct]);
          accK[jt][ct] = mfma(sa.hi, tr_frag(Qp + 32 * KLD, KLD, 4 * g, 16 + 4 * g, 16 * ct), accK[jt][ct]);
        }
      }
    }
    // dQs = dS Kt: dS^T (hi, lo) into the wave's tile, then read back by transposed reads
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jt = 0; jt < TM; ++jt) {
        bf16x4 h, l;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          __bf16 x, y;
          split1(df[rt][jt][r], x, y);
          h[r] = x;
          l[r] = y;
        }
        const int o = (16 * jt + c16) * SLD + 16 * rt + 4 * g;
        *reinterpret_cast<bf16x4*>(Sh + o) = h;
        *reinterpret_cast<bf16x4*>(Sl + o) = l;
      }
    // formed transposed, C^T(channel 16 ct + 4g + r, token 16 rt + lane % 16),
    // so a lane stores 4 consecutive channels of one token at once
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KM; ++kk) {
          const int k0 = 32 * kk + 8 * g;
          Frag2 sa, kb;
          sa.hi = tr_frag(Sh, SLD, k0, k0 + 4, 16 * rt);
          sa.lo = tr_frag(Sl, SLD, k0, k0 + 4, 16 * rt);
          kb.hi = tr_frag(Kh, KLD, k0, k0 + 4, 16 * ct);
          kb.lo = tr_frag(Kl, KLD, k0, k0 + 4, 16 * ct);
          c = mma<3>(kb, sa, c);
        }
        const int tok = ts + 16 * rt + c16;
        if (tok < t1)
          *reinterpret_cast<float4*>(a.dqf + ((size_t)bh * a.n + tok) * D + 16 * ct + 4 * g) =
              make_float4(c[0], c[1], c[2], c[3]);
      }
  }

  // the four waves' sums, added in wave order in LDS ([M][D] floats), then
  // written as the chunk's partials (dKt scaled by d^-1/4 here)
  float* const red = reinterpret_cast<float*>(t2_lds);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();  // LDS free (token loop done) / previous pass stored
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (wave == w) {
#pragma unroll
        for (int jt = 0; jt < TM; ++jt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float* const p = red + (16 * jt + 4 * g + r) * D + 16 * ct + c16;
              const float v = pass == 0 ? accW[jt][ct][r] : a.s4 * accK[jt][ct][r];
              *p = w == 0 ? v : *p + v;
            }
      }
      __syncthreads();
    }
    float* const dst = (pass == 0 ? a.pw : a.pk) + ((size_t)bh * a.nct + chunk) * M * D;
    for (int i = 4 * threadIdx.x; i < M * D; i += 4 * 256)
      *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(red + i);
  }
}

// ---------------------------------------------------------------------------
constexpr int BWD_MM_NT = 1024;  // threads of the per-head kernels (16 waves)

// LDS barrier without the global-memory drain of __syncthreads(): the
// kernels below keep global stores (the iteration's history) and prefetch
// loads in flight across it; only LDS writes must be complete.
__device__ __forceinline__ void lds_sync() {
  wait_lgkm0();
  barrier_only();
}

// Sum of the nch chunk partials p[ch * stride + i] for the four consecutive
// elements i .. i + 3 (16-byte aligned), in chunk order; up to 8 loads in
// flight per tensor.
__device__ __forceinline__ float4 sum_chunks4(const float* p, size_t stride, int nch) {
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += 8) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = c0 + u < nch ? *reinterpret_cast<const float4*>(p + (size_t)(c0 + u) * stride)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += x[u].x;
      s.y += x[u].y;
      s.z += x[u].z;
      s.w += x[u].w;
    }
  }
  return s;
}

// dW and dKt (F part) of one head from the token-chunk partials: each
// thread sums four consecutive elements over the chunks, in chunk order.
template <int M, int D>
__device__ __forceinline__ void reduce_token_partials(const BwdArgs& a, int bh, float* dW) {
  for (int i = 4 * threadIdx.x; i < M * D; i += 4 * BWD_MM_NT) {
    const size_t off = (size_t)bh * a.nct * M * D + i;
    *reinterpret_cast<float4*>(dW + i) = sum_chunks4(a.pw + off, (size_t)M * D, a.nct);
    *reinterpret_cast<float4*>(a.dKt + (size_t)bh * M * D + i) = sum_chunks4(a.pk + off, (size_t)M * D, a.nct);
  }
}


// Block-wide product C = alpha op(A) op(B) + beta C for float32 row-major
// matrices in global memory: op(A) is R x K, op(B) is K x N; each operand
// is staged in LDS (row stride + 4) first.  BWD_MM_NT threads.
template <int R, int N, int K>
__device__ void bgemm(float* C, const float* Ag, bool ta, const float* Bg, bool tb, float alpha, float beta,
                      float* La, float* Lb) {
  constexpr int NT = BWD_MM_NT, NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // stored shapes: A is (ta ? K x R : R x K), B is (tb ? N x K : K x N)
  const int ar = ta ? K : R, ac = ta ? R : K, br = tb ? N : K, bc = tb ? K : N;
  const int lda = ac + 4, ldb = bc + 4;
  __syncthreads();  // earlier results written; LDS free
  for (int i = threadIdx.x; i < ar * ac; i += NT) La[(i / ac) * lda + i % ac] = Ag[i];
  for (int i = threadIdx.x; i < br * bc; i += NT) Lb[(i / bc) * ldb + i % bc] = Bg[i];
  __syncthreads();
  const int ai = ta ? 1 : lda, ak = ta ? lda : 1;
  const int bk = tb ? 1 : ldb, bj = tb ? ldb : 1;
  constexpr int TR = R / 16, TN = N / 16;
  for (int t = wave; t < TR * TN; t += NWV) {
    const int it = t / TN, jt = t % TN;
    const f32x4 c = mm16<K>(La + 16 * it * ai, ai, ak, Lb + 16 * jt * bj, bk, bj, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* p = C + (size_t)(16 * it + 4 * g + r) * N + 16 * jt + c16;
      *p = beta == 0.f ? alpha * c[r] : alpha * c[r] + beta * *p;
    }
  }
}

// Above 128 landmarks the two whole operands no longer fit in LDS: the same
// product with the contraction taken in steps of KC, each step's slices of
// op(A) (R x KC) and op(B) (KC x N) staged in LDS, and every wave's C tiles
// held in registers across the steps.
constexpr int BWD_KC = 32;

template <int R, int N, int K>
__device__ void bgemm_kt(float* C, const float* Ag, bool ta, const float* Bg, bool tb, float alpha, float beta,
                         float* La, float* Lb) {
  constexpr int NT = BWD_MM_NT, NWV = NT / 64, KC = BWD_KC;
  constexpr int TR = R / 16, TN = N / 16, TILES = TR * TN, TPW = (TILES + NWV - 1) / NWV;
  constexpr int LDA = KC + 4, LDB = N + 4;
  static_assert(K % KC == 0, "whole contraction steps");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += KC) {
    __syncthreads();  // earlier results written; the previous step's reads done
    // stored shapes: A is (ta ? K x R : R x K), B is (tb ? N x K : K x N)
    for (int i = tid; i < R * KC; i += NT) {
      int r, kk;
      float x;
      if (ta) {
        kk = i / R, r = i % R;
        x = Ag[(size_t)(k0 + kk) * R + r];
      } else {
        r = i / KC, kk = i % KC;
        x = Ag[(size_t)r * K + k0 + kk];
      }
      La[r * LDA + kk] = x;
    }
    for (int i = tid; i < KC * N; i += NT) {
      int kk, j;
      float x;
      if (tb) {
        j = i / KC, kk = i % KC;
        x = Bg[(size_t)j * K + k0 + kk];
      } else {
        kk = i / N, j = i % N;
        x = Bg[(size_t)(k0 + kk) * N + j];
      }
      Lb[kk * LDB + j] = x;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + NWV * u;
      if (t < TILES)
        acc[u] = mm16<KC>(La + 16 * (t / TN) * LDA, LDA, 1, Lb + 16 * (t % TN), LDB, 1, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + NWV * u;
    if (t >= TILES) continue;
    const int it = t / TN, jt = t % TN;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* p = C + (size_t)(16 * it + 4 * g + r) * N + 16 * jt + c16;
      *p = beta == 0.f ? alpha * acc[u][r] : alpha * acc[u][r] + beta * *p;
    }
  }
}

// two staged operands of up to max(M, D) x max(M, D) floats (row stride + 4),
// or above 128 landmarks one contraction step of each (bgemm_kt)
template <int M, int D>
constexpr int bwd_mm_side() {
  return M > D ? M : D;
}
template <int M, int D>
constexpr bool bwd_mm_tiled() {
  return bwd_mm_side<M, D>() > 128;
}
template <int M, int D>
constexpr int bwd_mm_lds_bytes() {
  return bwd_mm_tiled<M, D>() ? 4 * (bwd_mm_side<M, D>() * (BWD_KC + 4) + BWD_KC * (bwd_mm_side<M, D>() + 4))
                              : 4 * 2 * bwd_mm_side<M, D>() * (bwd_mm_side<M, D>() + 4);
}

// The per-head product of the chain kernels: whole operands in LDS, or in
// contraction steps where they do not fit.
template <int R, int N, int K, int M, int D>
__device__ __forceinline__ void bgemm_h(float* C, const float* Ag, bool ta, const float* Bg, bool tb, float alpha,
                                        float beta, float* La, float* Lb) {
  if constexpr (bwd_mm_tiled<M, D>())
    bgemm_kt<R, N, K>(C, Ag, ta, Bg, tb, alpha, beta, La, Lb);
  else
    bgemm<R, N, K>(C, Ag, ta, Bg, tb, alpha, beta, La, Lb);
}

// A's maximum column sum with its column, and its maximum row sum (head bh).
// BWD_MM_NT threads.
template <int M>
__device__ void mm1_stats(const BwdArgs& a, int bh, const float* A) {
  constexpr int NT = BWD_MM_NT;
  const int tid = threadIdx.x;
  __shared__ float red[NT];
  __shared__ int redj[NT];
  float cs = -1.f, rs = 0.f;
  int cj = 0;
  if (tid < M) {
    cs = 0.f;
    for (int r = 0; r < M; ++r) cs += A[r * M + tid];
    for (int j = 0; j < M; ++j) rs += A[tid * M + j];
    cj = tid;
  }
  red[tid] = cs;
  redj[tid] = cj;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s && (red[tid + s] > red[tid] || (red[tid + s] == red[tid] && redj[tid + s] < redj[tid]))) {
      red[tid] = red[tid + s];
      redj[tid] = redj[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.cmax[bh] = red[0];
    a.cmaxj[bh] = redj[0];
  }
  __syncthreads();
  red[tid] = tid < M ? rs : 0.f;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  if (tid == 0) a.rmax[bh] = red[0];
}

// The end of the pseudo-inverse backward of head bh, given the gradient g
// reaching Z_0 = A^T / c: dA += g^T / c, dc = -sum(g A^T) / c^2, and A's
// statistics (mm1_stats).  BWD_MM_NT threads; g and dA are written before
// the call.
template <int M>
__device__ void mm1_tail(const BwdArgs& a, int bh, const float* A, const float* g, float* dA, float c) {
  constexpr int MM = M * M, NT = BWD_MM_NT;
  const int tid = threadIdx.x;
  float part = 0.f;
  for (int i = tid; i < MM; i += NT) {
    const int r = i / M, col = i % M;
    dA[i] += g[col * M + r] / c;
    part += g[col * M + r] * A[i];
  }
  __shared__ float dred[NT];
  dred[tid] = part;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) dred[tid] += dred[tid + s];
    __syncthreads();
  }
  if (tid == 0) a.dc[bh] = -dred[0] / (c * c);
  __syncthreads();
  mm1_stats<M>(a, bh, A);
}

// grid BH, block BWD_MM_NT, dynamic LDS bwd_mm_lds_bytes<M, D>().
template <int M, int D>
__global__ __launch_bounds__(BWD_MM_NT) void k_bwd_mm1(BwdArgs a) {
  constexpr int NT = BWD_MM_NT;
  extern __shared__ __align__(16) float bw_lds[];
  constexpr int MM = M * M;
  const int bh = blockIdx.x, tid = threadIdx.x;
  float* const La = bw_lds;
  float* const Lb = bw_lds + (bwd_mm_tiled<M, D>() ? bwd_mm_side<M, D>() * (BWD_KC + 4)
                                                    : bwd_mm_side<M, D>() * (bwd_mm_side<M, D>() + 4));
  const float* A = a.A + (size_t)bh * MM;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  auto Zk = [&](int k) { return S + (size_t)k * MM; };
  auto Xk = [&](int k) { return S + (size_t)(a.n_iter + 1 + 3 * k) * MM; };
  auto X2k = [&](int k) { return Xk(k) + MM; };
  auto Pk = [&](int k) { return Xk(k) + 2 * MM; };
  float* const G = S + (size_t)(4 * a.n_iter + 1) * MM;
  float* const Gn = G + MM;
  float* const dP = G + 2 * MM;
  float* const dX = G + 3 * MM;
  float* const T = G + 4 * MM;
  float* const dA = G + 5 * MM;
  float* const dW = a.dW + (size_t)bh * M * D;
  const float c = a.cscale[bh];

  // dW and dKt (F part) from the token-chunk partials, in chunk order
  reduce_token_partials<M, D>(a, bh, dW);
  // the iteration again in float32: Z_0 = A^T / c, X = A Z, P = 13I - 15X +
  // 7X^2 - X^3, Z <- Z P / 4; dA starts at zero
  for (int i = tid; i < MM; i += NT) {
    Zk(0)[i] = A[(i % M) * M + i / M] / c;
    dA[i] = 0.f;
  }
  for (int k = 0; k < a.n_iter; ++k) {
    bgemm_h<M, M, M, M, D>(Xk(k), A, false, Zk(k), false, 1.f, 0.f, La, Lb);
    bgemm_h<M, M, M, M, D>(X2k(k), Xk(k), false, Xk(k), false, 1.f, 0.f, La, Lb);
    bgemm_h<M, M, M, M, D>(Pk(k), Xk(k), false, X2k(k), false, -1.f, 0.f, La, Lb);
    __syncthreads();
    for (int i = tid; i < MM; i += NT)
      Pk(k)[i] += (i / M == i % M ? 13.f : 0.f) - 15.f * Xk(k)[i] + 7.f * X2k(k)[i];
    bgemm_h<M, M, M, M, D>(Zk(k + 1), Zk(k), false, Pk(k), false, 0.25f, 0.f, La, Lb);
  }
  // dZ_n = dW BV^T, dBV = Z_n^T dW
  bgemm_h<M, M, D, M, D>(G, dW, false, a.BV + (size_t)bh * M * D, true, 1.f, 0.f, La, Lb);
  bgemm_h<M, D, M, M, D>(a.dBV + (size_t)bh * M * D, Zk(a.n_iter), true, dW, false, 1.f, 0.f, La, Lb);
  float* g = G;
  float* gn = Gn;
  for (int k = a.n_iter - 1; k >= 0; --k) {
    float* const Z = Zk(k);
    float* const X = Xk(k);
    float* const X2 = X2k(k);
    bgemm_h<M, M, M, M, D>(gn, g, false, Pk(k), true, 0.25f, 0.f, La, Lb);   // dZ_k = G P^T / 4
    bgemm_h<M, M, M, M, D>(dP, Z, true, g, false, 0.25f, 0.f, La, Lb);        // dP = Z^T G / 4
    __syncthreads();
    for (int i = tid; i < MM; i += NT) dX[i] = -15.f * dP[i];
    bgemm_h<M, M, M, M, D>(dX, dP, false, X, true, 7.f, 1.f, La, Lb);         // + 7 dP X^T
    bgemm_h<M, M, M, M, D>(dX, X, true, dP, false, 7.f, 1.f, La, Lb);         // + 7 X^T dP
    bgemm_h<M, M, M, M, D>(dX, dP, false, X2, true, -1.f, 1.f, La, Lb);       // - dP (X^2)^T
    bgemm_h<M, M, M, M, D>(T, X, true, dP, false, 1.f, 0.f, La, Lb);
    bgemm_h<M, M, M, M, D>(dX, T, false, X, true, -1.f, 1.f, La, Lb);         // - X^T dP X^T
    bgemm_h<M, M, M, M, D>(dX, X2, true, dP, false, -1.f, 1.f, La, Lb);       // - (X^2)^T dP
    bgemm_h<M, M, M, M, D>(dA, dX, false, Z, true, 1.f, 1.f, La, Lb);         // dA += dX Z^T
    bgemm_h<M, M, M, M, D>(gn, A, true, dX, false, 1.f, 1.f, La, Lb);         // dZ_k += A^T dX
    float* const t = g;
    g = gn;
    gn = t;
  }
  __syncthreads();
  mm1_tail<M>(a, bh, A, g, dA, c);
}

// ---------------------------------------------------------------------------
// Above 64 landmarks the pseudo-inverse backward runs as a chain of launches
// over every head at once instead of one workgroup per head: each launch is
// one or two independent products (the same for all heads), each output a
// sum of up to four products plus elementwise terms,
//   C = sum_t alpha_t op(A_t) op(B_t) + beta C + g1 E1 + g2 E2 + eye I,
// with float32 row-major matrices, head h's at base + h * stride.  A
// workgroup of four waves forms one 32 x 32 tile of one output (a 16 x 16
// tile per wave); the 32-row strips of op(A) and op(B)^T over the whole
// contraction are staged in LDS per product.
struct ChainTerm {
  const float* a;
  const float* b;
  long long sa, sb;   // per-head strides (floats)
  int ta, tb;         // op = transpose
  int lda, ldb;       // stored row strides
  float alpha;
};
struct ChainOut {
  float* c;
  const float* e1;    // same shape and strides as C, or null
  const float* e2;
  long long sc;
  int R, N, K, ldc, nt;
  float beta, g1, g2, eye;
  ChainTerm t[4];
};
struct ChainLaunch {
  ChainOut o[2];
  int tiles0;         // workgroups of output 0; the rest are output 1's
};

__host__ __device__ constexpr int chain_tiles(int R, int N) { return ((R + 31) / 32) * ((N + 31) / 32); }
template <int KMAX>
constexpr int chain_lds_bytes() {
  return 2 * 32 * (KMAX + 4) * 4;
}

// Rows [r0, r0 + 32) of op(X) (K columns) into dst[32][K + 4]; X is stored
// K x rows (trans) or rows x K, row stride ld.  Rows at or past nrows are
// skipped (no wave reads them).  chain_load takes a thread's K / 32 16-byte
// pieces into registers, chain_store puts them in LDS, so both operands'
// loads are in flight together.
template <int KMAX>
__device__ __forceinline__ void chain_load(float4 (&v)[KMAX / 32], const float* x, int ld, bool trans, int r0,
                                           int nrows, int K) {
  const int tid = threadIdx.x, npc = 8 * K, k4 = K / 4;  // pieces: 32 rows x K / 4
#pragma unroll
  for (int u = 0; u < KMAX / 32; ++u) {
    const int i = tid + 256 * u;
    if (!trans) {
      const int rr = i / k4, kq = i % k4;
      if (i < npc && r0 + rr < nrows) v[u] = *reinterpret_cast<const float4*>(x + (size_t)(r0 + rr) * ld + 4 * kq);
    } else {
      // eight lanes per stored row (32 consecutive floats), one row per k
      const int rq = i % 8, k = i / 8;
      if (i < npc && r0 + 4 * rq < nrows) v[u] = *reinterpret_cast<const float4*>(x + (size_t)k * ld + r0 + 4 * rq);
    }
  }
}
template <int KMAX>
__device__ __forceinline__ void chain_store(float* dst, const float4 (&v)[KMAX / 32], bool trans, int r0, int nrows,
                                            int K, int ldl) {
  const int tid = threadIdx.x, npc = 8 * K, k4 = K / 4;
#pragma unroll
  for (int u = 0; u < KMAX / 32; ++u) {
    const int i = tid + 256 * u;
    if (!trans) {
      const int rr = i / k4, kq = i % k4;
      if (i < npc && r0 + rr < nrows) *reinterpret_cast<float4*>(dst + rr * ldl + 4 * kq) = v[u];
    } else {
      const int rq = i % 8, k = i / 8;
      if (i < npc && r0 + 4 * rq < nrows) {
        dst[(4 * rq + 0) * ldl + k] = v[u].x;
        dst[(4 * rq + 1) * ldl + k] = v[u].y;
        dst[(4 * rq + 2) * ldl + k] = v[u].z;
        dst[(4 * rq + 3) * ldl + k] = v[u].w;
      }
    }
  }
}

// grid (tiles of output 0 + tiles of output 1, BH), block 256, dynamic LDS
// chain_lds_bytes<KMAX>().
template <int KMAX>
__global__ __launch_bounds__(256) void k_bwd_chain(ChainLaunch L) {
  extern __shared__ __align__(16) float bw_lds[];
  constexpr int LDL = KMAX + 4;
  float* const As = bw_lds;
  float* const Bs = bw_lds + 32 * LDL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  const bool second = (int)blockIdx.x >= L.tiles0;
  const ChainOut& o = second ? L.o[1] : L.o[0];
  const int tile = (int)blockIdx.x - (second ? L.tiles0 : 0);
  const int tn = (o.N + 31) / 32;
  const int r0 = 32 * (tile / tn), c0 = 32 * (tile % tn);
  const int it = wave >> 1, jt = wave & 1;
  const bool live = r0 + 16 * it < o.R && c0 + 16 * jt < o.N;
  const int K = o.K;
  f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < o.nt; ++t) {
    const ChainTerm& tm = o.t[t];
    float4 va[KMAX / 32], vb[KMAX / 32];
    chain_load<KMAX>(va, tm.a + (size_t)bh * tm.sa, tm.lda, tm.ta != 0, r0, o.R, K);
    chain_load<KMAX>(vb, tm.b + (size_t)bh * tm.sb, tm.ldb, tm.tb == 0, c0, o.N, K);
    __syncthreads();  // the previous product's reads done
    chain_store<KMAX>(As, va, tm.ta != 0, r0, o.R, K, LDL);
    chain_store<KMAX>(Bs, vb, tm.tb == 0, c0, o.N, K, LDL);
    __syncthreads();
    if (live) {
      const float* pa = As + (16 * it + c16) * LDL + g;
      const float* pb = Bs + (16 * jt + c16) * LDL + g;
      f32x4 acc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K is a multiple of 16: four accumulators, one per k step mod 4
      for (int s = 0; s < K / 4; s += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_f32(pa[4 * (s + u)], pb[4 * (s + u)], acc[u]);
      }
      const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      tot += tm.alpha * sum;
    }
  }
  if (!live) return;
  float* const C = o.c + (size_t)bh * o.sc;
  const float* const E1 = o.e1 != nullptr ? o.e1 + (size_t)bh * o.sc : nullptr;
  const float* const E2 = o.e2 != nullptr ? o.e2 + (size_t)bh * o.sc : nullptr;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = r0 + 16 * it + 4 * g + r, col = c0 + 16 * jt + c16;
    const size_t i = (size_t)row * o.ldc + col;
    float v = tot[r];
    if (o.beta != 0.f) v += o.beta * C[i];
    if (E1 != nullptr) v += o.g1 * E1[i];
    if (E2 != nullptr) v += o.g2 * E2[i];
    if (row == col) v += o.eye;
    C[i] = v;
  }
}

// Start of the chain (it needs only A and c): Z_0 = A^T / c and dA = 0.
// grid (ceil(M M / 256), BH), block 256.
template <int M>
__global__ __launch_bounds__(256) void k_bwd_chain_init(BwdArgs a) {
  constexpr int MM = M * M;
  const int bh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  if (e < MM) {
    S[e] = a.A[(size_t)bh * MM + (e % M) * M + e / M] / a.cscale[bh];
    S[(size_t)(4 * a.n_iter + 1 + 5) * MM + e] = 0.f;  // dA
  }
}

// dW and dKt (F part) from the token-chunk partials: wave p of a workgroup
// sums chunks p, p + 4, p + 8, ... (in that order) of 64 four-element
// groups, then the four sums are added in wave order.  grid
// (ceil(M D / 256), BH), block 256.
template <int M, int D>
__global__ __launch_bounds__(256) void k_bwd_chain_sum(BwdArgs a) {
  constexpr int MD = M * D, NP = 4;
  __shared__ float4 part[NP][2][64];
  const int bh = blockIdx.y, lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int q = 4 * (blockIdx.x * 64 + lane);  // first element of the group
  float4 sw = make_float4(0.f, 0.f, 0.f, 0.f), sk = sw;
  if (q < MD) {
    const size_t off = ((size_t)bh * a.nct + p) * MD + q;
    const int cnt = (a.nct - p + NP - 1) / NP;
    sw = sum_chunks4(a.pw + off, (size_t)NP * MD, cnt);
    sk = sum_chunks4(a.pk + off, (size_t)NP * MD, cnt);
  }
  part[p][0][lane] = sw;
  part[p][1][lane] = sk;
  __syncthreads();
  if (p < 2 && q < MD) {
    float4 t = part[0][p][lane];
#pragma unroll
    for (int u = 1; u < NP; ++u) {
      const float4 x = part[u][p][lane];
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    *reinterpret_cast<float4*>((p == 0 ? a.dW : a.dKt) + (size_t)bh * MD + q) = t;
  }
}

// A's statistics for the chain (they need only A).  grid BH, block
// BWD_MM_NT.
template <int M>
__global__ __launch_bounds__(BWD_MM_NT) void k_bwd_chain_stats(BwdArgs a) {
  mm1_stats<M>(a, blockIdx.x, a.A + (size_t)blockIdx.x * M * M);
}

// End of the chain, with g the gradient reaching Z_0 (matrix gsel of the
// scratch, the G or Gn slot): dA += g^T / c over 32 x 32 tiles (g's tile
// transposed through LDS), and per tile the partial sum of g^T * A for dc
// (into the dX slot, which the chain no longer needs).  grid ((M / 32)^2,
// BH), block 256.
template <int M>
__global__ __launch_bounds__(256) void k_bwd_chain_post(BwdArgs a, int gsel) {
  constexpr int MM = M * M, TPR = M / 32;
  static_assert(M % 32 == 0, "whole 32 x 32 tiles");
  __shared__ float tg[32][33];
  __shared__ float red[256];
  const int bh = blockIdx.y, tid = threadIdx.x, blk = blockIdx.x;
  const int r0 = 32 * (blk / TPR), c0 = 32 * (blk % TPR);
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  const float* const g = S + (size_t)gsel * MM;
  float* const dA = S + (size_t)(4 * a.n_iter + 1 + 5) * MM;
  const float* const A = a.A + (size_t)bh * MM;
  const float c = a.cscale[bh];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e, y = idx / 32, x = idx % 32;
    tg[y][x] = g[(size_t)(c0 + y) * M + r0 + x];
  }
  __syncthreads();
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e, y = idx / 32, x = idx % 32;
    const size_t i = (size_t)(r0 + y) * M + c0 + x;
    const float gv = tg[x][y];  // g[c0 + x][r0 + y]
    dA[i] += gv / c;
    part += gv * A[i];
  }
  red[tid] = part;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) S[(size_t)(4 * a.n_iter + 1 + 3) * MM + blk] = red[0];
}

// dc = -sum(g A^T) / c^2 from the tiles' partial sums, in tile order.
// grid BH, block 64.
template <int M>
__global__ __launch_bounds__(64) void k_bwd_chain_dc(BwdArgs a) {
  constexpr int MM = M * M, NB = (M / 32) * (M / 32);
  const int bh = blockIdx.x;
  const float* const p = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM + (size_t)(4 * a.n_iter + 1 + 3) * MM;
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int i = 0; i < NB; ++i) s += p[i];
    const float c = a.cscale[bh];
    a.dc[bh] = -s / (c * c);
  }
}

// Product on operands already in LDS (row strides lda, ldb; flat
// pointers), C = alpha op(A) op(B) + beta C with C in LDS or global memory
// (row stride ldc).  Starts with an LDS barrier (operands written, C free).
template <int R, int N, int K>
__device__ void lgemm(float* C, int ldc, const float* La, int lda, bool ta, const float* Lb, int ldb, bool tb,
                      float alpha, float beta) {
  constexpr int NWV = BWD_MM_NT / 64, TR = R / 16, TN = N / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  lds_sync();
  const int ai = ta ? 1 : lda, ak = ta ? lda : 1;
  const int bk = tb ? 1 : ldb, bj = tb ? ldb : 1;
  for (int t = wave; t < TR * TN; t += NWV) {
    const int it = t / TN, jt = t % TN;
    const f32x4 c = mm16<K>(La + 16 * it * ai, ai, ak, Lb + 16 * jt * bj, bk, bj, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* p = C + (size_t)(16 * it + 4 * g + r) * ldc + 16 * jt + c16;
      *p = beta == 0.f ? alpha * c[r] : alpha * c[r] + beta * *p;
    }
  }
}

// The calling wave's tile (it, jt) = (wave / 4, wave % 4) of a 64 x 64
// product on LDS operands, added to acc (16 waves: one tile each).
__device__ __forceinline__ f32x4 ltile64(const float* La, int lda, bool ta, const float* Lb, int ldb, bool tb,
                                         f32x4 acc) {
  const int wave = threadIdx.x >> 6, it = wave >> 2, jt = wave & 3;
  lds_sync();
  const int ai = ta ? 1 : lda, ak = ta ? lda : 1;
  const int bk = tb ? 1 : ldb, bj = tb ? ldb : 1;
  return mm16<64>(La + 16 * it * ai, ai, ak, Lb + 16 * jt * bj, bk, bj, acc);
}

// LDS image of a row-major M x Mc global matrix (row stride ld).
__device__ __forceinline__ void lds_load(float* dst, int ld, const float* src, int M, int Mc) {
  lds_sync();
  for (int i = threadIdx.x; i < M * Mc; i += BWD_MM_NT) dst[(i / Mc) * ld + i % Mc] = src[i];
}
__device__ __forceinline__ void lds_store(float* dst, const float* src, int ld, int M, int Mc) {
  lds_sync();
  for (int i = threadIdx.x; i < M * Mc; i += BWD_MM_NT) dst[i] = src[(i / Mc) * ld + i % Mc];
}

constexpr int BWD_MM64_LDS = 4 * 6 * 64 * 68;

// The forward half of the 64-landmark per-head chain: the iteration again
// in float32 (Z_0 = A^T / c, X = A Z, X^2, P = 13I - 15X + 7X^2 - X^3,
// Z <- Z P / 4) with the history Z_k, X_k, X_k^2, P_k written to the
// per-head scratch for k_bwd_mm1b64, and A's largest column sum (its first
// column) and largest row sum.  It needs only A, so it runs beside the
// token pass.  A, Z, X, X^2, P and a spare slot as float32 images in LDS
// (row stride 68), 16 waves.
// grid BH, block BWD_MM_NT, dynamic LDS BWD_MM64_LDS.
static __global__ __launch_bounds__(BWD_MM_NT) void k_bwd_mm1f64(BwdArgs a) {
  extern __shared__ __align__(16) float bw_lds[];
  constexpr int M = 64, MM = M * M, LD = M + 4, SZ = M * LD, NT = BWD_MM_NT;
  const int bh = blockIdx.x, tid = threadIdx.x;
  float* const sA = bw_lds;
  float* sZ = sA + SZ;
  float* sG = sZ + SZ;  // spare slot
  float* const sX = sG + SZ;
  float* const sX2 = sX + SZ;
  float* const sPT = sX2 + SZ;
  const float* A = a.A + (size_t)bh * MM;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  auto Zk = [&](int k) { return S + (size_t)k * MM; };
  auto Xk = [&](int k) { return S + (size_t)(a.n_iter + 1 + 3 * k) * MM; };
  auto X2k = [&](int k) { return Xk(k) + MM; };
  auto Pk = [&](int k) { return Xk(k) + 2 * MM; };
  const float c = a.cscale[bh];

  lds_load(sA, LD, A, M, M);
  lds_sync();
  for (int i = tid; i < MM; i += NT) {
    const float z = sA[(i % M) * LD + i / M] / c;
    sZ[(i / M) * LD + i % M] = z;
    Zk(0)[i] = z;
  }
  for (int k = 0; k < a.n_iter; ++k) {
    lgemm<M, M, M>(sX, LD, sA, LD, false, sZ, LD, false, 1.f, 0.f);
    lgemm<M, M, M>(sX2, LD, sX, LD, false, sX, LD, false, 1.f, 0.f);
    lgemm<M, M, M>(sPT, LD, sX, LD, false, sX2, LD, false, -1.f, 0.f);
    lds_sync();
    for (int i = tid; i < MM; i += NT) {
      const int o = (i / M) * LD + i % M;
      sPT[o] += (i / M == i % M ? 13.f : 0.f) - 15.f * sX[o] + 7.f * sX2[o];
      Xk(k)[i] = sX[o];
      X2k(k)[i] = sX2[o];
      Pk(k)[i] = sPT[o];
    }
    lgemm<M, M, M>(sG, LD, sZ, LD, false, sPT, LD, false, 0.25f, 0.f);  // Z_{k+1} (into the spare slot)
    lds_store(Zk(k + 1), sG, LD, M, M);
    float* const t = sZ;
    sZ = sG;
    sG = t;
  }
  // A's largest column sum (the first such column) and largest row sum
  lds_sync();
  float* const red = sX;
  int* const redj = reinterpret_cast<int*>(sX2);
  float cs = -1.f, rs = 0.f;
  int cj = 0;
  if (tid < M) {
    cs = 0.f;
    for (int r = 0; r < M; ++r) cs += sA[r * LD + tid];
    for (int j = 0; j < M; ++j) rs += sA[tid * LD + j];
    cj = tid;
  }
  red[tid] = cs;
  redj[tid] = cj;
  __syncthreads();
  for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2 && (red[tid + s2] > red[tid] || (red[tid + s2] == red[tid] && redj[tid + s2] < redj[tid]))) {
      red[tid] = red[tid + s2];
      redj[tid] = redj[tid + s2];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.cmax[bh] = red[0];
    a.cmaxj[bh] = redj[0];
  }
  __syncthreads();
  red[tid] = tid < M ? rs : 0.f;
  __syncthreads();
  for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] = fmaxf(red[tid], red[tid + s2]);
    __syncthreads();
  }
  if (tid == 0) a.rmax[bh] = red[0];
}

// The backward half of the 64-landmark per-head chain in float32 (float32
// I/O): the products of k_bwd_mm1b64 on the float32 matrix cores over
// float32 images of A, G, G', dP, dX, Z_k, X_k, X_k^2 and P_k (then T) in
// LDS (row stride 68); the history comes back one step at a time (the four
// matrices of a step in one batch of loads) and each wave keeps its 16 x 16
// tile of dA in registers.  Once the iteration has converged a relative
// error e in its products grows to about e cond(A), so float32 I/O keeps
// float32 products here as in the forward iteration.
// grid BH, block BWD_MM_NT, dynamic LDS BWD_MM64B_LDS.
constexpr int BWD_MM64B_LDS = 4 * 9 * 64 * 68;
template <int D>
__global__ __launch_bounds__(BWD_MM_NT) void k_bwd_mm1b64_f32(BwdArgs a) {
  extern __shared__ __align__(16) float bw_lds[];
  constexpr int M = 64, MM = M * M, LD = M + 4, SZ = M * LD, NT = BWD_MM_NT;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  float* const sA = bw_lds;
  float* sG = sA + SZ;
  float* sGn = sG + SZ;
  float* const sdP = sGn + SZ;
  float* const sdX = sdP + SZ;
  float* sZ = sdX + SZ;
  float* const sX = sZ + SZ;
  float* const sX2 = sX + SZ;
  float* const sPT = sX2 + SZ;
  const float* A = a.A + (size_t)bh * MM;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  auto Zk = [&](int k) { return S + (size_t)k * MM; };
  auto Xk = [&](int k) { return S + (size_t)(a.n_iter + 1 + 3 * k) * MM; };
  auto X2k = [&](int k) { return Xk(k) + MM; };
  auto Pk = [&](int k) { return Xk(k) + 2 * MM; };
  float* const dA = S + (size_t)(4 * a.n_iter + 1 + 5) * MM;
  float* const dW = a.dW + (size_t)bh * M * D;
  const float c = a.cscale[bh];

  reduce_token_partials<M, D>(a, bh, dW);
  lds_load(sA, LD, A, M, M);
  lds_load(sZ, LD, Zk(a.n_iter), M, M);
  // dZ_n = dW BV^T and dBV = Z_n^T dW, with dW and BV staged in the dP and
  // dX slots (for D = 128, rows of D + 4 floats: dW across the dP and dX
  // slots, BV across the X and X^2 slots, which the loop below reloads)
  constexpr int LDW = D <= M ? LD : D + 4;
  static_assert(M * LDW <= 2 * SZ, "dW and BV fit two slots");
  float* const sW = sdP;
  float* const sBV = D <= M ? sdX : sX;
  lds_load(sW, LDW, dW, M, D);
  lds_load(sBV, LDW, a.BV + (size_t)bh * M * D, M, D);
  lgemm<M, M, D>(sG, LD, sW, LDW, false, sBV, LDW, true, 1.f, 0.f);
  lgemm<M, D, M>(a.dBV + (size_t)bh * M * D, D, sZ, LD, true, sW, LDW, false, 1.f, 0.f);
  // the history stores are complete before any of it is read back
  wait_vmcnt<0>();
  f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};  // this wave's tile of dA
  for (int k = a.n_iter - 1; k >= 0; --k) {
    {
      // Z_k, X_k, X_k^2, P_k into LDS: every load of the step in flight at once
      constexpr int PER = MM / NT;
      float hz[PER], hx[PER], hx2[PER], hp[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = tid + u * NT;
        hz[u] = Zk(k)[i];
        hx[u] = Xk(k)[i];
        hx2[u] = X2k(k)[i];
        hp[u] = Pk(k)[i];
      }
      lds_sync();
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = tid + u * NT, o = (i / M) * LD + i % M;
        sZ[o] = hz[u];
        sX[o] = hx[u];
        sX2[o] = hx2[u];
        sPT[o] = hp[u];
      }
    }
    lgemm<M, M, M>(sGn, LD, sG, LD, false, sPT, LD, true, 0.25f, 0.f);   // dZ_k = G P^T / 4
    lgemm<M, M, M>(sdP, LD, sZ, LD, true, sG, LD, false, 0.25f, 0.f);    // dP = Z^T G / 4
    lds_sync();
    for (int i = tid; i < MM; i += NT) {
      const int o = (i / M) * LD + i % M;
      sdX[o] = -15.f * sdP[o];
    }
    lgemm<M, M, M>(sdX, LD, sdP, LD, false, sX, LD, true, 7.f, 1.f);     // + 7 dP X^T
    lgemm<M, M, M>(sdX, LD, sX, LD, true, sdP, LD, false, 7.f, 1.f);     // + 7 X^T dP
    lgemm<M, M, M>(sdX, LD, sdP, LD, false, sX2, LD, true, -1.f, 1.f);   // - dP (X^2)^T
    lgemm<M, M, M>(sPT, LD, sX, LD, true, sdP, LD, false, 1.f, 0.f);     // T = X^T dP
    lgemm<M, M, M>(sdX, LD, sPT, LD, false, sX, LD, true, -1.f, 1.f);    // - X^T dP X^T
    lgemm<M, M, M>(sdX, LD, sX2, LD, true, sdP, LD, false, -1.f, 1.f);   // - (X^2)^T dP
    dacc = ltile64(sdX, LD, false, sZ, LD, true, dacc);                   // dA += dX Z^T
    lgemm<M, M, M>(sGn, LD, sA, LD, true, sdX, LD, false, 1.f, 1.f);     // dZ_k += A^T dX
    float* const t = sG;
    sG = sGn;
    sGn = t;
  }
  lds_sync();
  // Z_0 = A^T / c: dA += G^T / c, written with the wave's tile; dc = -sum(G A^T) / c^2
  float part = 0.f;
  {
    const int it = wave >> 2, jt = wave & 3, col = 16 * jt + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * it + 4 * g + r;
      const float gv = sG[col * LD + row];
      dA[row * M + col] = dacc[r] + gv / c;
      part += gv * sA[row * LD + col];
    }
  }
  float* const red = sX;  // free now
  red[tid] = part;
  __syncthreads();
  for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] += red[tid + s2];
    __syncthreads();
  }
  if (tid == 0) a.dc[bh] = -red[0] / (c * c);
}

// ---------------------------------------------------------------------------
// The backward half of the 64-landmark per-head chain on the bf16 matrix
// cores (bf16 I/O).  Every 64 x 64 operand lives in LDS as split-bf16 hi / lo planes
// (row-major, row stride PL_LD), so a product of two of them is six
// v_mfma_f32_16x16x32_bf16 per 16 x 16 tile; each of the 16 waves owns one
// output tile (it, jt) = (wave / 4, wave % 4) of every product and keeps
// the running sums (dZ_k, dX, dA) in float32 registers.  Operand access:
// "row" reads 8 consecutive k of a row (an operand Y, or Y^T on the right),
// "tr" reads 8 consecutive k of a column by transposed reads (Y^T on the
// left, Y on the right).  The history Z_k, X_k, X_k^2, P_k comes from
// k_bwd_mm1f in float32 and is split as it is staged, one step ahead.
constexpr int PL_LD = 64 + 8;                 // bf16 row stride of a plane
constexpr int PL_MAT = 2 * 64 * PL_LD;        // elements of one split matrix
constexpr int BWD_MM1B_LDS = 8 * PL_MAT * 2;  // eight split matrices (bytes)

// C tile (16 it.., 16 jt..) += op(X) op(Y) over k < 64, op(X) = X (row) or
// X^T (TX, tr), op(Y) = Y^T (row) or Y (TY, tr); planes hi at p, lo at p + 64 PL_LD.
template <bool TX, bool TY>
__device__ __forceinline__ f32x4 pmm(const __bf16* X, const __bf16* Y, int it, int jt, f32x4 acc) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int k0 = 32 * ks + 8 * g;
    Frag2 a, b;
    if constexpr (TX) {
      a.hi = tr_frag(X, PL_LD, k0, k0 + 4, 16 * it);
      a.lo = tr_frag(X + 64 * PL_LD, PL_LD, k0, k0 + 4, 16 * it);
    } else {
      a.hi = *reinterpret_cast<const bf16x8*>(X + (16 * it + c16) * PL_LD + k0);
      a.lo = *reinterpret_cast<const bf16x8*>(X + 64 * PL_LD + (16 * it + c16) * PL_LD + k0);
    }
    if constexpr (TY) {
      b.hi = tr_frag(Y, PL_LD, k0, k0 + 4, 16 * jt);
      b.lo = tr_frag(Y + 64 * PL_LD, PL_LD, k0, k0 + 4, 16 * jt);
    } else {
      b.hi = *reinterpret_cast<const bf16x8*>(Y + (16 * jt + c16) * PL_LD + k0);
      b.lo = *reinterpret_cast<const bf16x8*>(Y + 64 * PL_LD + (16 * jt + c16) * PL_LD + k0);
    }
    acc = mma<3>(a, b, acc);
  }
  return acc;
}

// The wave's C tile (rows 16 it + 4g + r, column 16 jt + c16) into a split matrix.
__device__ __forceinline__ void put_tile(__bf16* Y, int it, int jt, f32x4 v) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 h, l;
    split1(v[r], h, l);
    const int o = (16 * it + 4 * g + r) * PL_LD + 16 * jt + c16;
    Y[o] = h;
    Y[64 * PL_LD + o] = l;
  }
}

// Four consecutive elements (4 threadIdx.x .. + 3 of a row-major float32
// 64 x 64 matrix) into a split matrix.
__device__ __forceinline__ void put4(__bf16* Y, float4 v) {
  const int i = 4 * threadIdx.x, row = i >> 6, col = i & 63;
  const float x[4] = {v.x, v.y, v.z, v.w};
  bf16x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __bf16 a, b;
    split1(x[e], a, b);
    h[e] = a;
    l[e] = b;
  }
  *reinterpret_cast<bf16x4*>(Y + row * PL_LD + col) = h;
  *reinterpret_cast<bf16x4*>(Y + 64 * PL_LD + row * PL_LD + col) = l;
}

// grid BH, block BWD_MM_NT, dynamic LDS BWD_MM1B_LDS.
template <int D>
__global__ __launch_bounds__(BWD_MM_NT) void k_bwd_mm1b64(BwdArgs a) {
  extern __shared__ __align__(16) __bf16 pl_lds[];
  constexpr int M = 64, MM = M * M, LD = M + 4, SZ = M * LD, NT = BWD_MM_NT;
  static_assert(4 * NT == MM, "one float4 of each matrix per thread");
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int it = wave >> 2, jt = wave & 3;
  const float* A = a.A + (size_t)bh * MM;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  auto Zk = [&](int k) { return S + (size_t)k * MM; };
  auto Xk = [&](int k) { return S + (size_t)(a.n_iter + 1 + 3 * k) * MM; };
  auto X2k = [&](int k) { return Xk(k) + MM; };
  auto Pk = [&](int k) { return Xk(k) + 2 * MM; };
  float* const dA = S + (size_t)(4 * a.n_iter + 1 + 5) * MM;
  float* const dW = a.dW + (size_t)bh * M * D;
  const float c = a.cscale[bh];
  __bf16* const pA = pl_lds;
  __bf16* const pG = pA + PL_MAT;
  __bf16* const pdP = pG + PL_MAT;
  __bf16* const pdX = pdP + PL_MAT;
  __bf16* const pZ = pdX + PL_MAT;
  __bf16* const pX = pZ + PL_MAT;
  __bf16* const pX2 = pX + PL_MAT;
  __bf16* const pPT = pX2 + PL_MAT;  // P_k, then T

  // ---- setup in float32 (the LDS is used as float32 images first):
  // dW, dZ_n = G = dW BV^T, dBV = Z_n^T dW
  float* const fl = reinterpret_cast<float*>(pl_lds);
  constexpr int LDW = D <= M ? LD : D + 4;
  float* const sZ = fl;
  float* const sG = sZ + SZ;
  float* const sW = sG + SZ;
  float* const sBV = sW + M * LDW;
  static_assert(4 * (2 * SZ + 2 * M * LDW) <= BWD_MM1B_LDS, "setup images fit");
  reduce_token_partials<M, D>(a, bh, dW);
  lds_load(sZ, LD, Zk(a.n_iter), M, M);
  lds_load(sW, LDW, dW, M, D);
  lds_load(sBV, LDW, a.BV + (size_t)bh * M * D, M, D);
  lgemm<M, M, D>(sG, LD, sW, LDW, false, sBV, LDW, true, 1.f, 0.f);
  lgemm<M, D, M>(a.dBV + (size_t)bh * M * D, D, sZ, LD, true, sW, LDW, false, 1.f, 0.f);
  lds_sync();
  f32x4 gt;  // the wave's tile of G (float32)
#pragma unroll
  for (int r = 0; r < 4; ++r) gt[r] = sG[(16 * it + 4 * g + r) * LD + 16 * jt + c16];
  // the first step's history and A, as split matrices (after every wave's
  // read of the float32 images)
  float4 hz = make_float4(0.f, 0.f, 0.f, 0.f), hx = hz, hx2 = hz, hp = hz;
  const float4 av = *reinterpret_cast<const float4*>(A + 4 * tid);
  if (a.n_iter > 0) {
    const int k = a.n_iter - 1;
    hz = *reinterpret_cast<const float4*>(Zk(k) + 4 * tid);
    hx = *reinterpret_cast<const float4*>(Xk(k) + 4 * tid);
    hx2 = *reinterpret_cast<const float4*>(X2k(k) + 4 * tid);
    hp = *reinterpret_cast<const float4*>(Pk(k) + 4 * tid);
  }
  lds_sync();
  put4(pA, av);
  put_tile(pG, it, jt, gt);

  f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = a.n_iter - 1; k >= 0; --k) {
    lds_sync();  // the last step's reads of Z, X, X^2, T are done
    put4(pZ, hz);
    put4(pX, hx);
    put4(pX2, hx2);
    put4(pPT, hp);
    if (k > 0) {
      hz = *reinterpret_cast<const float4*>(Zk(k - 1) + 4 * tid);
      hx = *reinterpret_cast<const float4*>(Xk(k - 1) + 4 * tid);
      hx2 = *reinterpret_cast<const float4*>(X2k(k - 1) + 4 * tid);
      hp = *reinterpret_cast<const float4*>(Pk(k - 1) + 4 * tid);
    }
    lds_sync();
    const f32x4 z0 = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 gn = pmm<false, false>(pG, pPT, it, jt, z0) * 0.25f;  // dZ_k = G P^T / 4 ...
    const f32x4 dp = pmm<true, true>(pZ, pG, it, jt, z0) * 0.25f;  // dP = Z^T G / 4
    put_tile(pdP, it, jt, dp);
    lds_sync();
    const f32x4 t = pmm<true, true>(pX, pdP, it, jt, z0);  // T = X^T dP
    f32x4 dx = -15.f * dp + 7.f * pmm<false, false>(pdP, pX, it, jt, z0) + 7.f * t -
               pmm<false, false>(pdP, pX2, it, jt, z0);
    put_tile(pPT, it, jt, t);  // P's readers (the first product) are a barrier back
    lds_sync();
    dx -= pmm<false, false>(pPT, pX, it, jt, z0) + pmm<true, true>(pX2, pdP, it, jt, z0);  // - T X^T - (X^2)^T dP
    put_tile(pdX, it, jt, dx);
    lds_sync();
    dacc = pmm<false, false>(pdX, pZ, it, jt, dacc);  // dA += dX Z^T
    gn = pmm<true, true>(pA, pdX, it, jt, gn);        // ... + A^T dX
    gt = gn;
    put_tile(pG, it, jt, gt);  // G's last readers (the two products at the top) are two barriers back
  }
  // Z_0 = A^T / c: dA += G^T / c (G in float32 through LDS); dc = -sum(G A^T) / c^2
  lds_sync();
  float* const gf = fl;  // [64][LD] float32, over the planes (all reads done)
#pragma unroll
  for (int r = 0; r < 4; ++r) gf[(16 * it + 4 * g + r) * LD + 16 * jt + c16] = gt[r];
  lds_sync();
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * it + 4 * g + r, col = 16 * jt + c16;
    const float gv = gf[col * LD + row];
    dA[row * M + col] = dacc[r] + gv / c;
    part += gv * A[row * M + col];
  }
  float* const red = fl + SZ;
  red[tid] = part;
  __syncthreads();
  for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] += red[tid + s2];
    __syncthreads();
  }
  if (tid == 0) a.dc[bh] = -red[0] / (c * c);
}

// grid BH, block BWD_MM_NT, dynamic LDS bwd_mm_lds_bytes<M, D>().  Row
// work runs 16 threads to a row (a row's 16 threads are 16 consecutive
// lanes, reduced with sum16).
template <int M, int D, bool CHAINED = false>
__global__ __launch_bounds__(BWD_MM_NT) void k_bwd_mm2(BwdArgs a) {
  constexpr int NT = BWD_MM_NT;
  extern __shared__ __align__(16) float bw_lds[];
  constexpr int MM = M * M, RPP = NT / 16;
  const int bh = blockIdx.x, tid = threadIdx.x, l16 = tid & 15;
  float* const La = bw_lds;
  float* const Lb = bw_lds + (bwd_mm_tiled<M, D>() ? bwd_mm_side<M, D>() * (BWD_KC + 4)
                                                    : bwd_mm_side<M, D>() * (bwd_mm_side<M, D>() + 4));
  const float* A = a.A + (size_t)bh * MM;
  float* const S = a.mm + (size_t)bh * bwd_mm_mats(a.n_iter) * MM;
  const float* const dA = S + (size_t)(4 * a.n_iter + 1 + 5) * MM;
  float* const dSA = S + (size_t)(4 * a.n_iter + 1 + 4) * MM;  // the T slot
  // c's share, added to column j* of dA: for option 0 only in the head
  // holding the maximum column sum over all heads (the first such head),
  // with the sum of every head's dc and the largest row sum
  float add;
  if (a.init_option == 0) {
    __shared__ float rsum[NT], rmx[NT], rbest[NT];
    __shared__ int rh[NT];
    float sdc = 0.f, srm = 0.f, best = -INFINITY;
    int hb = 0x7fffffff;
    for (int h = tid; h < a.BH; h += NT) {
      sdc += a.dc[h];
      srm = fmaxf(srm, a.rmax[h]);
      const float cm = a.cmax[h];
      if (cm > best) {
        best = cm;
        hb = h;
      }
    }
    rsum[tid] = sdc;
    rmx[tid] = srm;
    rbest[tid] = best;
    rh[tid] = hb;
    __syncthreads();
    for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
      if (tid < s2) {
        rsum[tid] += rsum[tid + s2];
        rmx[tid] = fmaxf(rmx[tid], rmx[tid + s2]);
        if (rbest[tid + s2] > rbest[tid] || (rbest[tid + s2] == rbest[tid] && rh[tid + s2] < rh[tid])) {
          rbest[tid] = rbest[tid + s2];
          rh[tid] = rh[tid + s2];
        }
      }
      __syncthreads();
    }
    add = rh[0] == bh ? rsum[0] * rmx[0] : 0.f;
  } else {
    add = a.dc[bh] * a.rmax[bh];
  }
  const int jstar = a.cmaxj[bh];
  // dS_A = A (dA - rowsum(dA A))
  for (int r = tid / 16; r < M; r += RPP) {
    float av[M / 16], dv[M / 16];
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < M / 16; ++u) {
      const int j = l16 + 16 * u;
      av[u] = A[r * M + j];
      dv[u] = dA[r * M + j] + (j == jstar ? add : 0.f);
      s += dv[u] * av[u];
    }
    s = sum16(s);
#pragma unroll
    for (int u = 0; u < M / 16; ++u) dSA[r * M + l16 + 16 * u] = av[u] * (dv[u] - s);
  }
  // dQt_A = dS_A Kt; dKt += dS_A^T Qt (bgemm starts with a block barrier;
  // CHAINED: one k_bwd_chain launch over all heads after this kernel)
  if constexpr (!CHAINED) {
    bgemm_h<M, D, M, M, D>(a.dQt + (size_t)bh * M * D, dSA, false, a.kt + (size_t)bh * M * D, false, 1.f, 0.f, La,
                           Lb);
    bgemm_h<M, D, M, M, D>(a.dKt + (size_t)bh * M * D, dSA, true, a.qt + (size_t)bh * M * D, false, 1.f, 1.f, La,
                           Lb);
  }
  // D_i = dBV_i . BV_i
  for (int r = tid / 16; r < M; r += RPP) {
    const float* x = a.dBV + ((size_t)bh * M + r) * D;
    const float* y = a.BV + ((size_t)bh * M + r) * D;
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) s += x[l16 + 16 * u] * y[l16 + 16 * u];
    s = sum16(s);
    if (l16 == 0) a.Dv[(size_t)bh * M + r] = s;
  }
}

// ---------------------------------------------------------------------------
template <int M, int D>
struct BwdKeyLayout {
  static constexpr int LDB = BWD_GK + 4, LD = D + 4;
  // above 128 landmarks the pass takes the landmarks in two halves of MH
  // rows (Qt, dBV and the B / dS tiles of one half in LDS at a time); the
  // first half's dv / dk contributions go to a float32 buffer and come back,
  // to the lane that wrote them, in the second
  static constexpr int NHALF = M > 128 ? 2 : 1;
  static constexpr int MH = NHALF == 1 ? M : (M / 2 + 15) / 16 * 16;
  static constexpr int OFF_QT = 0;
  static constexpr int OFF_DBV = OFF_QT + MH * LD;
  static constexpr int OFF_KS = OFF_DBV + MH * LD;
  static constexpr int OFF_V = OFF_KS + BWD_GK * LD;
  static constexpr int OFF_B = OFF_V + BWD_GK * LD;
  static constexpr int OFF_DS = OFF_B + MH * LDB;
  static constexpr int OFF_VAL = OFF_DS + MH * LDB;
  // key-major copies of B (in B's area) and dS for the bf16 dv / dk products
  static constexpr int LDT = MH + 4;
  static constexpr int OFF_DST = OFF_VAL + BWD_GK;
  static constexpr int FLOATS = OFF_DST + BWD_GK * LDT;
  static constexpr int BYTES = 4 * FLOATS;
  static_assert(BYTES <= 160 * 1024, "k_bwd_key LDS");
  static_assert(BWD_GK * LDT <= MH * LDB, "the key-major B fits in B's area");
  static_assert(NHALF * MH >= M, "the halves cover every landmark");
};

constexpr int BWD_KEY_NT = 512;  // threads of k_bwd_key (8 waves)

// grid (nck, BH), block BWD_KEY_NT.
template <typename IO, int M, int D>
__global__ __launch_bounds__(BWD_KEY_NT) void k_bwd_key(BwdArgs a) {
  constexpr int NT = BWD_KEY_NT, NWV = NT / 64;
  extern __shared__ __align__(16) float bw_lds[];
  using Ly = BwdKeyLayout<M, D>;
  constexpr int NH = Ly::NHALF, MH = Ly::MH, TH = MH / 16, CT = D / 16, LDB = Ly::LDB, LD = Ly::LD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x, b = bh / a.H;
  const int ck = bwd_key_chunk(M, D);
  const int k0 = chunk * ck, k1 = min(a.n, k0 + ck);
  const IO* Kg = reinterpret_cast<const IO*>(a.k) + (size_t)bh * a.n * D;
  const IO* Vg = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  const float* lse = a.lse + (size_t)bh * M;
  const float* Dv = a.Dv + (size_t)bh * M;
  const float* dKt = a.dKt + (size_t)bh * M * D;
  float* const Qt = bw_lds + Ly::OFF_QT;
  float* const dBV = bw_lds + Ly::OFF_DBV;
  float* const Ks = bw_lds + Ly::OFF_KS;
  float* const Vs = bw_lds + Ly::OFF_V;
  float* const Bt = bw_lds + Ly::OFF_B;
  float* const DS = bw_lds + Ly::OFF_DS;
  float* const VAL = bw_lds + Ly::OFF_VAL;
  // the first half's dv, then dk, contributions ([BH][n][D] each)
  float* const hv = a.dvk;
  float* const hk = a.dvk != nullptr ? a.dvk + (size_t)a.BH * a.n * D : nullptr;
  const float inv_l = 1.0f / (float)a.L;
  // at bf16 I/O, S, dB and dQt_B run on the bf16 matrix cores: k (staged
  // unscaled; S and the dQt_B partials take the d^-1/4 instead) and v are
  // exact bf16 operands, Qt, dBV and dS split hi + lo (relative error about
  // 2^-16); dv and dk stay on float32 products
  constexpr bool BF = sizeof(IO) == 2;
  const float ks = BF ? 1.f : a.s4;  // the scale staged with k
  // dv and dk on bf16 products as well where the half is whole 32-landmark
  // blocks: B and dS also stored key-major (BtT, DST), and each wave's fixed
  // channel tile of dBV and Qt split into fragments once per half
  constexpr bool BFV = BF && MH % 32 == 0 && D == 64;
  constexpr int LDT = Ly::LDT, NKB = BFV ? MH / 32 : 1;
  float* const BtT = Bt;  // B's area
  float* const DST = bw_lds + Ly::OFF_DST;
  static_assert(!BFV || 2 * (BWD_GK / 16) * CT == 2 * NWV, "a dv and a dk tile per wave, same key and channel tile");
  // dQt_B tiles (landmark tile of the half, channel tile) owned by this wave: t = wave + NWV j
  constexpr int NACC = (TH * CT + NWV - 1) / NWV;
  for (int h = 0; h < NH; ++h) {
    const int i0 = h * MH;  // the half's first landmark; rows at or past M are zero
    __syncthreads();        // the previous half's reads done
    for (int i = tid; i < MH * D; i += NT) {
      const int r = i / D, c = i % D;
      const bool in = i0 + r < M;
      Qt[r * LD + c] = in ? a.qt[((size_t)bh * M + i0 + r) * D + c] : 0.f;
      dBV[r * LD + c] = in ? a.dBV[((size_t)bh * M + i0 + r) * D + c] : 0.f;
    }
    f32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag2 fbv[NKB], fbq[NKB];  // B(landmark 32 kb + 8g + e, channel 16 ct + c16) of dBV and Qt
    if constexpr (BFV) {
      __syncthreads();  // the half staged
      const int ctw = wave % CT;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float xv[8], xq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xv[e] = dBV[(32 * kb + 8 * g + e) * LD + 16 * ctw + c16];
          xq[e] = Qt[(32 * kb + 8 * g + e) * LD + 16 * ctw + c16];
        }
        fbv[kb] = split8(xv);
        fbq[kb] = split8(xq);
      }
    }
    for (int gk = k0; gk < k1; gk += BWD_GK) {
      __syncthreads();  // staging done / previous step's reads done
      static_assert(BWD_GK * (D / 8) <= NT, "one chunk of K and of V per thread");
      if (tid < BWD_GK * (D / 8)) {
        // one 8-element chunk of K and of V per thread
        const int r = tid / (D / 8), c = 8 * (tid % (D / 8)), key = gk + r;
        float xk[8], xv[8];
        if (key < k1) {
          IOTraits<IO>::load8(Kg + (size_t)key * D + c, xk);
          IOTraits<IO>::load8(Vg + (size_t)key * D + c, xv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xk[e] = xv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          Ks[r * LD + c + e] = xk[e] * ks;
          Vs[r * LD + c + e] = xv[e];
        }
      }
      if (tid < BWD_GK) {
        const int key = gk + tid;
        VAL[tid] = (key < k1 && (mask == nullptr || mask[key] != 0)) ? 1.f : 0.f;
      }
      __syncthreads();
      // B (from the stored normalisers) and dS_B = B (dBV V^T - D_i): C(landmark, key)
      for (int t = wave; t < TH * (BWD_GK / 16); t += NWV) {
        const int it = t / (BWD_GK / 16), kt = t % (BWD_GK / 16);
        f32x4 s, db;
        if constexpr (BF) {
          // A(landmark c16, channel 32 kb + 8g + e), B(channel, key c16)
          s = db = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb) {
            const int ch = 32 * kb + 8 * g;
            const Frag2 fq = split8(Qt + (16 * it + c16) * LD + ch);
            const Frag2 fd = split8(dBV + (16 * it + c16) * LD + ch);
            bf16x8 bk, bv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              bk[e] = (__bf16)Ks[(16 * kt + c16) * LD + ch + e];
              bv[e] = (__bf16)Vs[(16 * kt + c16) * LD + ch + e];
            }
            s = mfma(fq.hi, bk, s);
            s = mfma(fq.lo, bk, s);
            db = mfma(fd.hi, bv, db);
            db = mfma(fd.lo, bv, db);
          }
          s *= a.s4;
        } else {
          s = mm16<D>(Qt + 16 * it * LD, LD, 1, Ks + 16 * kt * LD, 1, LD, f32x4{0.f, 0.f, 0.f, 0.f});
          db = mm16<D>(dBV + 16 * it * LD, LD, 1, Vs + 16 * kt * LD, 1, LD, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        const float val = VAL[16 * kt + c16];
        float bq[4], dq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int il = 16 * it + 4 * g + r, i = i0 + il;
          const bool on = val != 0.f && i < M;
          bq[r] = on ? exp2f(s[r] * LOG2E - lse[i]) : 0.f;
          dq[r] = i < M ? bq[r] * (db[r] - Dv[i]) : 0.f;
          if constexpr (!BFV) Bt[il * LDB + 16 * kt + c16] = bq[r];
          DS[il * LDB + 16 * kt + c16] = dq[r];
        }
        if constexpr (BFV) {
          // key-major: the lane's four landmarks 16 it + 4g + r are consecutive
          const int o = (16 * kt + c16) * LDT + 16 * it + 4 * g;
          *reinterpret_cast<float4*>(BtT + o) = make_float4(bq[0], bq[1], bq[2], bq[3]);
          *reinterpret_cast<float4*>(DST + o) = make_float4(dq[0], dq[1], dq[2], dq[3]);
        }
      }
      __syncthreads();
      // dv = B^T dBV + dv_conv and dk = d^-1/4 (dS^T Qt + dKt[seg] / L): C(key, channel)
      for (int t = wave; t < 2 * (BWD_GK / 16) * CT; t += NWV) {
        const bool isk = t >= (BWD_GK / 16) * CT;
        const int tt = t % ((BWD_GK / 16) * CT), kt = tt / CT, ct = tt % CT;
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BFV) {
          // A(key c16, landmark 32 kb + 8g + e) from the key-major copies
          const float* const at = (isk ? DST : BtT) + (16 * kt + c16) * LDT + 8 * g;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) c = mma<3>(split8(at + 32 * kb), isk ? fbq[kb] : fbv[kb], c);
        } else {
          c = mm16<MH>((isk ? DS : Bt) + 16 * kt, 1, LDB, (isk ? Qt : dBV) + 16 * ct, LD, 1, c);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = gk + 16 * kt + 4 * g + r, ch = 16 * ct + c16;
          if (key >= k1) continue;
          const size_t o = ((size_t)bh * a.n + key) * D + ch;
          float x = c[r];
          if constexpr (NH == 2) {
            if (h == 0) {
              (isk ? hk : hv)[o] = x;
              continue;
            }
            x = (isk ? hk : hv)[o] + x;
          }
          if (isk) {
            x += dKt[(size_t)(key / a.L) * D + ch] * inv_l;
            io_put(reinterpret_cast<IO*>(a.dk) + o, a.s4 * x);
          } else {
            x += a.dvc != nullptr ? a.dvc[o] : 0.f;
            io_put(reinterpret_cast<IO*>(a.dv) + o, x);
          }
        }
      }
      // dQt_B += dS Ks: C(landmark, channel), summed over the step's keys
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        const int t = wave + NWV * j;
        if (t < TH * CT) {
          const int it = t / CT, ct = t % CT;
          if constexpr (BF) {
            // A(landmark c16, key 8g + e), B(key, channel c16)
            static_assert(BWD_GK == 32, "one 16 x 16 x 32 product per step");
            const Frag2 fs = split8(DS + (16 * it + c16) * LDB + 8 * g);
            bf16x8 bk;
#pragma unroll
            for (int e = 0; e < 8; ++e) bk[e] = (__bf16)Ks[(8 * g + e) * LD + 16 * ct + c16];
            acc[j] = mfma(fs.hi, bk, acc[j]);
            acc[j] = mfma(fs.lo, bk, acc[j]);
          } else {
            acc[j] = mm16<BWD_GK>(DS + 16 * it * LDB, LDB, 1, Ks + 16 * ct, LD, 1, acc[j]);
          }
        }
      }
    }
    float* const pq = a.pq + ((size_t)bh * a.nck + chunk) * M * D;
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      const int t = wave + NWV * j;
      if (t < TH * CT) {
        const int it = t / CT, ct = t % CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i0 + 16 * it + 4 * g + r;
          if (row < M) pq[(size_t)row * D + 16 * ct + c16] = (BF ? a.s4 : 1.f) * acc[j][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key pass on the bf16 matrix cores, for the shapes of k_bwd_tok2 (split
// hi / lo operands; k and v rows of bf16 I/O are exact).  Each wave works
// alone on 32-key steps (steps wave, wave + 4, ... of the chunk):
//   S = Qt Ks^T and dB = dBV v^T as C tiles (landmark 16 it + 4g + r, key
//   16 kt + lane % 16), B = exp2(S log2 e - lse) on kept keys, dS = B (dB -
//   D_i) (no cross-lane work: B's normalisers are stored);
//   dv = B^T dBV and dk = dS^T Qt: the contraction runs over landmarks in
//   the paired k order (two stacked landmark tiles), so B and dS enter as A
//   operands from registers, dBV and Qt as B operands by transposed reads;
//   dQt += dS Ks: dS^T goes to the wave's LDS tile, A by transposed reads,
//   summed over all of the wave's steps in registers; the four waves' sums
//   are added in wave order at the end.

template <typename IO, int M, int D>
struct BwdKey2Layout {
  static constexpr int NSK = sizeof(IO) == 2 ? 1 : 2;  // bf16 planes of the staged k / v rows
  static constexpr int KLD = D + 8;                    // element row stride of Qt, dBV, k, v tiles
  static constexpr int SLD = M + 8;                    // element row stride of the dS^T tile
  static constexpr int QT = 0;                    // Qt hi, lo [M][KLD]
  static constexpr int DB = QT + 2 * M * KLD;     // dBV hi, lo
  static constexpr int WAVE0 = DB + 2 * M * KLD;  // per-wave areas
  static constexpr int KW = 0;                    // k rows [32][KLD], NSK planes
  static constexpr int VW = KW + NSK * 32 * KLD;  // v rows
  static constexpr int SW = VW + NSK * 32 * KLD;  // dS^T hi, lo [32][SLD]
  static constexpr int PER_WAVE = SW + 2 * 32 * SLD;
  static constexpr int BYTES = 2 * (WAVE0 + 4 * PER_WAVE);
  static_assert(BYTES <= 160 * 1024, "k_bwd_key2 LDS");
  static_assert(4 * M * D <= BYTES, "the epilogue sums [M][D] floats in LDS");
};

// grid (ceil(n / BWD_K2_CK), BH), block 256, dynamic LDS BwdKey2Layout::BYTES.
template <typename IO, int M, int D>
__global__ __launch_bounds__(256) void k_bwd_key2(BwdArgs a) {
  extern __shared__ __align__(16) __bf16 k2_lds[];
  using Ly = BwdKey2Layout<IO, M, D>;
  constexpr int NSK = Ly::NSK, KLD = Ly::KLD, SLD = Ly::SLD;
  constexpr int TM = M / 16, CT = D / 16, KD = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x, b = bh / a.H;
  const int k0c = chunk * BWD_K2_CK, k1 = min(a.n, k0c + BWD_K2_CK);
  const IO* Kg = reinterpret_cast<const IO*>(a.k) + (size_t)bh * a.n * D;
  const IO* Vg = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  const float* dKt = a.dKt + (size_t)bh * M * D;
  __bf16* const Qh = k2_lds + Ly::QT;
  __bf16* const Ql = Qh + M * KLD;
  __bf16* const Bh = k2_lds + Ly::DB;
  __bf16* const Bl = Bh + M * KLD;
  __bf16* const wb = k2_lds + Ly::WAVE0 + wave * Ly::PER_WAVE;
  __bf16* const Kp = wb + Ly::KW;  // plane p at Kp + p * 32 * KLD
  __bf16* const Vp = wb + Ly::VW;
  __bf16* const Sh = wb + Ly::SW;
  __bf16* const Sl = Sh + 32 * SLD;

  // Qt and dBV (float32 [M][D]) as bf16 hi / lo planes
  for (int i = threadIdx.x; i < M * D / 8; i += 256) {
    const int r = i / (D / 8), c = 8 * (i % (D / 8));
    float x[8];
    IOTraits<float>::load8(a.qt + ((size_t)bh * M + r) * D + c, x);
    const Frag2 fq = split8(x);
    *reinterpret_cast<bf16x8*>(Qh + r * KLD + c) = fq.hi;
    *reinterpret_cast<bf16x8*>(Ql + r * KLD + c) = fq.lo;
    IOTraits<float>::load8(a.dBV + ((size_t)bh * M + r) * D + c, x);
    const Frag2 fb = split8(x);
    *reinterpret_cast<bf16x8*>(Bh + r * KLD + c) = fb.hi;
    *reinterpret_cast<bf16x8*>(Bl + r * KLD + c) = fb.lo;
  }
  // the lane's rows 16 it + 4g + r: B's log2 normalisers and D_i
  float lse[TM][4], dv_i[TM][4];
#pragma unroll
  for (int it = 0; it < TM; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * it + 4 * g + r;
      lse[it][r] = a.lse[(size_t)bh * M + i];
      dv_i[it][r] = a.Dv[(size_t)bh * M + i];
    }

  const int sr = lane >> 1, sc = (lane & 1) * (D / 2);
  const int nsteps = (k1 - k0c + 31) / 32;
  RowBuf<IO, D / 2> bk, bv;
  // per step, also the lane's mask bits, conv part of dv and dKt[segment]
  // elements (transposed C layout: key 16 kt + lane % 16, channels 16 ct +
  // 4g .. + 3, one 16-byte load each), fetched a step ahead with the k and v
  // rows
  bool pkeep[2];
  float4 pdvc[2][CT], pdkt[2][CT];
  auto fetch = [&](int step) {
    const int ks = k0c + 32 * step;
    {
      const int key = ks + sr;
      const bool ok = key < k1;
      const size_t o = (size_t)(ok ? key : k0c) * D + sc;
      bk.load(Kg + o, ok);
      bv.load(Vg + o, ok);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = ks + 16 * kt + c16;
      const bool ok = key < k1;
      pkeep[kt] = ok && (mask == nullptr || mask[key] != 0);
      const int seg = (ok ? key : k0c) / a.L;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int ch = 16 * ct + 4 * g;
        pdvc[kt][ct] = (ok && a.dvc != nullptr)
                           ? *reinterpret_cast<const float4*>(a.dvc + ((size_t)bh * a.n + key) * D + ch)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        pdkt[kt][ct] = *reinterpret_cast<const float4*>(dKt + (size_t)seg * D + ch);
      }
    }
  };
  if (wave < nsteps) fetch(wave);
  f32x4 accQ[TM][CT];
#pragma unroll
  for (int it = 0; it < TM; ++it)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) accQ[it][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float inv_l = 1.0f / (float)a.L;
  __syncthreads();  // Qt, dBV staged

  for (int step = wave; step < nsteps; step += 4) {
    const int ks0 = k0c + 32 * step;
    bk.store(Kp + sr * KLD + sc, Kp + 32 * KLD + sr * KLD + sc);
    bv.store(Vp + sr * KLD + sc, Vp + 32 * KLD + sr * KLD + sc);
    // this step's prefetched values, then the next step's fetch
    bool keep[2];
    float4 cdvc[2][CT], cdkt[2][CT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      keep[kt] = pkeep[kt];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        cdvc[kt][ct] = pdvc[kt][ct];
        cdkt[kt][ct] = pdkt[kt][ct];
      }
    }
    if (step + 4 < nsteps) fetch(step + 4);
    // S = Qt k^T (Qt carries d^-1/4; k gets it here) and dB = dBV v^T
    f32x4 s[TM][2], db[TM][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      Frag2 kb[KD], vb[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        const int o = (16 * kt + c16) * KLD + 32 * ks + 8 * g;
        kb[ks].hi = *reinterpret_cast<const bf16x8*>(Kp + o);
        vb[ks].hi = *reinterpret_cast<const bf16x8*>(Vp + o);
        if constexpr (NSK == 2) {
          kb[ks].lo = *reinterpret_cast<const bf16x8*>(Kp + 32 * KLD + o);
          vb[ks].lo = *reinterpret_cast<const bf16x8*>(Vp + 32 * KLD + o);
        }
      }
#pragma unroll
      for (int it = 0; it < TM; ++it) {
        f32x4 cs = f32x4{0.f, 0.f, 0.f, 0.f}, cd = cs;
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          const int o = (16 * it + c16) * KLD + 32 * ks + 8 * g;
          const bf16x8 qh = *reinterpret_cast<const bf16x8*>(Qh + o);
          const bf16x8 ql = *reinterpret_cast<const bf16x8*>(Ql + o);
          const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(Bh + o);
          const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(Bl + o);
          cs = mfma(qh, kb[ks].hi, cs);
          cs = mfma(ql, kb[ks].hi, cs);
          cd = mfma(bh_, vb[ks].hi, cd);
          cd = mfma(bl_, vb[ks].hi, cd);
          if constexpr (NSK == 2) {
            cs = mfma(qh, kb[ks].lo, cs);
            cd = mfma(bh_, vb[ks].lo, cd);
          }
        }
        // B and dS = B (dB - D_i), in place of s and db
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float bb = keep[kt] ? exp2f(cs[r] * a.s4 * LOG2E - lse[it][r]) : 0.f;
          s[it][kt][r] = bb;
          db[it][kt][r] = bb * (cd[r] - dv_i[it][r]);
        }
      }
    }
    // dv = B^T dBV + dv_conv and dk = d^-1/4 (dS^T Qt + dKt[segment] / L),
    // formed transposed: C^T(channel 16 ct + 4g + r, key 16 kt + lane % 16),
    // landmarks in the paired k order (B and dS, from registers, as the B
    // operand), so a lane stores 4 consecutive channels of one key
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 cv[CT], ck[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) cv[ct] = ck[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < TM / 2; ++p) {
        const float bx[8] = {s[2 * p][kt][0], s[2 * p][kt][1], s[2 * p][kt][2], s[2 * p][kt][3],
                             s[2 * p + 1][kt][0], s[2 * p + 1][kt][1], s[2 * p + 1][kt][2], s[2 * p + 1][kt][3]};
        const float sx[8] = {db[2 * p][kt][0], db[2 * p][kt][1], db[2 * p][kt][2], db[2 * p][kt][3],
                             db[2 * p + 1][kt][0], db[2 * p + 1][kt][1], db[2 * p + 1][kt][2], db[2 * p + 1][kt][3]};
        const Frag2 ba = split8(bx), sa = split8(sx);
        const int i0 = 32 * p + 4 * g, i1 = i0 + 16;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Frag2 dbv, qt;
          dbv.hi = tr_frag(Bh, KLD, i0, i1, 16 * ct);
          dbv.lo = tr_frag(Bl, KLD, i0, i1, 16 * ct);
          qt.hi = tr_frag(Qh, KLD, i0, i1, 16 * ct);
          qt.lo = tr_frag(Ql, KLD, i0, i1, 16 * ct);
          cv[ct] = mma<3>(dbv, ba, cv[ct]);
          ck[ct] = mma<3>(qt, sa, ck[ct]);
        }
      }
      const int key = ks0 + 16 * kt + c16;
      if (key < k1) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const size_t o = ((size_t)bh * a.n + key) * D + 16 * ct + 4 * g;
          const float4 dc = cdvc[kt][ct], kc = cdkt[kt][ct];
          io_put4(reinterpret_cast<IO*>(a.dv) + o,
                  f32x4{cv[ct][0] + dc.x, cv[ct][1] + dc.y, cv[ct][2] + dc.z, cv[ct][3] + dc.w});
          io_put4(reinterpret_cast<IO*>(a.dk) + o,
                  f32x4{a.s4 * (ck[ct][0] + kc.x * inv_l), a.s4 * (ck[ct][1] + kc.y * inv_l),
                        a.s4 * (ck[ct][2] + kc.z * inv_l), a.s4 * (ck[ct][3] + kc.w * inv_l)});
        }
      }
    }
    // dQt += dS k (times d^-1/4 at the end): dS^T (hi, lo) into the wave's
    // tile [key][landmark], A by transposed reads (k = key, 8g + e)
#pragma unroll
    for (int it = 0; it < TM; ++it)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x4 h, l;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          __bf16 x, y;
          split1(db[it][kt][r], x, y);
          h[r] = x;
          l[r] = y;
        }
        const int o = (16 * kt + c16) * SLD + 16 * it + 4 * g;
        *reinterpret_cast<bf16x4*>(Sh + o) = h;
        *reinterpret_cast<bf16x4*>(Sl + o) = l;
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      bf16x8 kbh = tr_frag(Kp, KLD, 8 * g, 8 * g + 4, 16 * ct), kbl;
      if constexpr (NSK == 2) kbl = tr_frag(Kp + 32 * KLD, KLD, 8 * g, 8 * g + 4, 16 * ct);
#pragma unroll
      for (int it = 0; it < TM; ++it) {
        const bf16x8 sh = tr_frag(Sh, SLD, 8 * g, 8 * g + 4, 16 * it);
        const bf16x8 sl = tr_frag(Sl, SLD, 8 * g, 8 * g + 4, 16 * it);
        accQ[it][ct] = mfma(sh, kbh, accQ[it][ct]);
        accQ[it][ct] = mfma(sl, kbh, accQ[it][ct]);
        if constexpr (NSK == 2) accQ[it][ct] = mfma(sh, kbl, accQ[it][ct]);
      }
    }
  }

  // the four waves' sums in wave order, then the chunk's partial of dQt
  float* const red = reinterpret_cast<float*>(k2_lds);
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int it = 0; it < TM; ++it)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* const p = red + (16 * it + 4 * g + r) * D + 16 * ct + c16;
            const float v = a.s4 * accQ[it][ct][r];
            *p = w == 0 ? v : *p + v;
          }
    }
    __syncthreads();
  }
  float* const dst = a.pq + ((size_t)bh * a.nck + chunk) * M * D;
  for (int i = 4 * threadIdx.x; i < M * D; i += 4 * 256)
    *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(red + i);
}

// dQt = dQt_A + sum of the key-chunk partials: a workgroup covers 256
// elements as 64 four-element groups; wave p sums chunks p, p + 4, p + 8,
// ... (in that order), then dQt_A and the four sums are added in wave
// order.  grid (M * D / 256, BH), block 256.
template <int M, int D>
__global__ __launch_bounds__(256) void k_bwd_qt(BwdArgs a) {
  constexpr int MD = M * D, NP = 4;
  __shared__ float4 part[NP][64];
  const int bh = blockIdx.y, lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int q = 4 * (blockIdx.x * 64 + lane);
  const int cnt = (a.nck - p + NP - 1) / NP;
  part[p][lane] = sum_chunks4(a.pq + ((size_t)bh * a.nck + p) * MD + q, (size_t)NP * MD, cnt);
  __syncthreads();
  if (p == 0) {
    float4* const dst = reinterpret_cast<float4*>(a.dQt + (size_t)bh * MD + q);
    float4 t = *dst;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const float4 x = part[u][lane];
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    *dst = t;
  }
}

// dq = d^-1/4 (dQs + dQt[segment] / L).  grid (ceil(n / 64), BH), block 256:
// thread = (token, quarter of the D channels).
template <typename IO, int M, int D>
__global__ __launch_bounds__(256) void k_bwd_q(BwdArgs a) {
  const int bh = blockIdx.y;
  const int tok = blockIdx.x * 64 + (threadIdx.x >> 2), c0 = (D / 4) * (threadIdx.x & 3);
  if (tok >= a.n) return;
  const float inv_l = 1.0f / (float)a.L;
  const float* dqf = a.dqf + ((size_t)bh * a.n + tok) * D + c0;
  const float* dqt = a.dQt + ((size_t)bh * M + tok / a.L) * D + c0;
  IO* const dq = reinterpret_cast<IO*>(a.dq) + ((size_t)bh * a.n + tok) * D + c0;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) io_put(dq + e, a.s4 * (dqf[e] + dqt[e] * inv_l));
}

// dv_conv[t] = sum_j w[j] dout[t - j + K/2]: the forward's convolution of
// dout with the taps reversed, on the matrix cores as three banded Toeplitz
// products per 16-token tile (the window of dout staged in LDS, transposed,
// bf16 hi/lo).  grid (ceil(n / 128), BH), block 256, dynamic LDS
// bwd_dv_lds<D>().
constexpr int BWD_DV_TOK = 128;
constexpr int BWD_DV_WIN = BWD_DV_TOK + 80;
constexpr int BWD_DV_LD = BWD_DV_WIN + 8;
template <int D>
constexpr int bwd_dv_lds() {
  return 2 * 2 * D * BWD_DV_LD + 4 * TAPS;
}

template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_dvconv(BwdArgs a) {
  extern __shared__ __align__(16) __bf16 dv_lds[];
  constexpr int NS = IOTraits<IO>::NS;
  __bf16* const vh = dv_lds;
  __bf16* const vl = vh + D * BWD_DV_LD;
  float* const wf = reinterpret_cast<float*>(vl + D * BWD_DV_LD);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15;
  const int bh = blockIdx.y, h = bh % a.H, t0 = blockIdx.x * BWD_DV_TOK, K = a.conv_k;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  stage_v_window<IO, D>(DO, D, a.n, t0, BWD_DV_WIN, vh, vl, BWD_DV_LD);
  if (threadIdx.x < K) wf[threadIdx.x] = a.conv_w[(size_t)h * K + K - 1 - threadIdx.x];
  __syncthreads();
  Frag2 tap[3];
  conv_taps(wf, K, tap);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;
    if (ts >= a.n) continue;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    conv_tile<NS, false, D>(vh, vl, BWD_DV_LD, ts - t0, tap, oacc);
    const int tok = ts + c16;
    if (tok < a.n) store_row16<float, false, D>(a.dvc + ((size_t)bh * a.n + tok) * D, oacc);
  }
}

// The chunk's partial dconv_w[j] = sum_t,c dout[t][c] v[t + j - K/2][c], on
// the matrix cores: per 16-token tile at ts, P = dout_tile V_win^T (16 x 96
// positions ts - 32 .. ts + 63, split-bf16 products), whose entry (t, s)
// belongs to tap j = s - 32 - t + K/2.  A lane's (column tile, row) slots map
// to the same taps in every tile, so each lane sums its slots over the
// workgroup's tiles in registers; the slots of each tap are then added in a
// fixed order.  grid (ncv, BH), block 256, dynamic LDS bwd_cv_lds<D>(): V
// window rows t0 - 32 .. t0 + 192 row-major as bf16 hi / lo planes, the
// 16-byte chunks of a row XOR-swizzled by its low row bits (cv_swz).
constexpr int BWD_CVWIN = BWD_CV + 96;
template <int D>
constexpr int bwd_cv_lds() {
  return 2 * 2 * BWD_CVWIN * D + 4 * (4 * 6 * 4 * 64);
}
template <int D>
__device__ __forceinline__ int cv_swz(int row, int chunk) {
  constexpr int MASK = (D / 8 < 8 ? D / 8 : 8) - 1;
  return row * D + 8 * (chunk ^ (row & MASK));
}

template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_conv(BwdArgs a) {
  extern __shared__ __align__(16) __bf16 cv_lds[];
  constexpr int NS = IOTraits<IO>::NS;
  __bf16* const vh = cv_lds;
  __bf16* const vl = vh + BWD_CVWIN * D;
  float* const red = reinterpret_cast<float*>(vl + BWD_CVWIN * D);  // [wave][st][r][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, chunk = blockIdx.x, t0 = chunk * BWD_CV, K = a.conv_k, half = K / 2;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const IO* V = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  // V window, row-major, 16-byte chunks swizzled by row
  for (int i = threadIdx.x; i < BWD_CVWIN * (D / 8); i += 256) {
    const int r = i / (D / 8), cc = i % (D / 8), t = t0 - HALO + r;
    float x[8];
    if (t >= 0 && t < a.n) {
      IOTraits<IO>::load8(V + (size_t)t * D + 8 * cc, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    const Frag2 f = make_frag<NS>(x);
    *reinterpret_cast<bf16x8*>(vh + cv_swz<D>(r, cc)) = f.hi;
    if constexpr (NS == 3) *reinterpret_cast<bf16x8*>(vl + cv_swz<D>(r, cc)) = f.lo;
  }
  __syncthreads();
  f32x4 acc[6];
#pragma unroll
  for (int st = 0; st < 6; ++st) acc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ts = t0 + 32 * wave + 16 * u;  // tile start
    if (ts >= a.n) continue;
    const int tok = ts + c16;
    constexpr int KS = D / 32;  // 32-channel steps of the products
    Frag2 df[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      if (tok < a.n) {
        IOTraits<IO>::load8(DO + (size_t)tok * D + 32 * ks + 8 * g, x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      df[ks] = make_frag<NS>(x);
    }
    // P^T tiles: C(position 16 st + 4 g + r, token c16) = sum_c V[pos][c] dout[tok][c]
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      const int row = ts - t0 + 16 * st + c16;  // window row of position ts - 32 + 16 st + c16
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag2 vf;
        vf.hi = *reinterpret_cast<const bf16x8*>(vh + cv_swz<D>(row, 4 * ks + g));
        if constexpr (NS == 3) vf.lo = *reinterpret_cast<const bf16x8*>(vl + cv_swz<D>(row, 4 * ks + g));
        acc[st] = mma<NS>(vf, df[ks], acc[st]);
      }
    }
  }
  // lane (c16 = token t, g) slot (st, r): position offset 16 st + 4 g + r - 32
  // from the tile start, tap j = 16 st + 4 g + r - 32 - c16 + half
#pragma unroll
  for (int st = 0; st < 6; ++st)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * 6 + st) * 4 + r) * 64 + lane] = acc[st][r];
  __syncthreads();
  if (threadIdx.x < K) {
    const int j = threadIdx.x;
    float sum = 0.f;
    // slot (st, gg, r) holds tap j for token cc = 16 st + base, base = 4 gg + r - 32 + half - j:
    // one column tile st per (gg, r)
    for (int w = 0; w < 4; ++w)
      for (int gg = 0; gg < 4; ++gg)
        for (int r = 0; r < 4; ++r) {
          const int base = 4 * gg + r - 32 + half - j;  // in [-96, 47]
          const int st = (111 - base) / 16 - 6;           // ceil(-base / 16) for base > -112
          const int cc = 16 * st + base;
          if (st >= 0 && st < 6 && cc < 16) sum += red[((w * 6 + st) * 4 + r) * 64 + 16 * gg + cc];
        }
    a.pconv[((size_t)bh * a.ncv + chunk) * K + j] = sum;
  }
}

// dconv_w[h][j] = sum over batches and chunks: 8 threads per tap each take
// every 8th partial, then the 8 sums are added in order.  grid H, block 1024.
static __global__ __launch_bounds__(1024) void k_bwd_wsum(BwdArgs a) {
  __shared__ float ps[8][TAPS];
  const int h = blockIdx.x, K = a.conv_k, j = threadIdx.x >> 3, p = threadIdx.x & 7;
  const int B = a.BH / a.H, cnt = B * a.ncv;
  if (j < K) {
    float s = 0.f;
    for (int i0 = p; i0 < cnt; i0 += 64) {
      float x[8];  // eight loads in flight, added in order
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 8 * u, b = i / a.ncv, ch = i % a.ncv;
        x[u] = i < cnt ? a.pconv[((size_t)(b * a.H + h) * a.ncv + ch) * K + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    ps[p][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    float s = 0.f;
    for (int q = 0; q < 8; ++q) s += ps[q][threadIdx.x];
    a.dconv_w[(size_t)h * K + threadIdx.x] = s;
  }
}

// ---------------------------------------------------------------------------
// Exact branch (m == n; page section 2.1): P = softmax(Qs Ks^T + mask),
// out = P V (+ conv).  Flash-style backward in three passes:
//   k_bwd_xstats  per query: lse (log2 units) and D_t = dout_t . (P V)_t;
//   k_bwd_xq      per query tile: dS = P (dout V^T - D), dq = s4 dS Ks;
//   k_bwd_xkv     per key tile: dv = P^T dout (+ dv_conv), dk = s4 dS^T Qs.
// P is recomputed from the stored lse, so every pass streams the other
// side in 32-row steps through LDS.

struct XBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const uint8_t* key_mask;
  const float* dvc;   // conv part of dv or null
  float* lse;         // [BH][n]
  float* Dt;          // [BH][n]
  void* dq;
  void* dk;
  void* dv;
  int n, H;
  float s4;
};

constexpr int XB_T = 64;   // rows of the tile a workgroup owns (4 waves x 16)
constexpr int XB_S = 32;   // rows of the streamed side per step

// Stage rows [r0, r0 + R) of X (scaled) into LDS [R][D + 4] with 256
// threads, one 8-element chunk per thread and step; rows past n are zero.
template <typename IO, int D, int R>
__device__ __forceinline__ void xb_rows(const IO* X, int r0, int n, float scale, float* dst) {
  constexpr int CPR = D / 8;
  static_assert((R * CPR) % 256 == 0 || R * CPR < 256, "whole steps");
#pragma unroll
  for (int u = 0; u < (R * CPR + 255) / 256; ++u) {
    const int i = threadIdx.x + 256 * u, r = i / CPR, c = 8 * (i % CPR);
    if (i >= R * CPR) break;
    float x[8];
    if (r0 + r < n) {
      IOTraits<IO>::load8(X + (size_t)(r0 + r) * D + c, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[r * (D + 4) + c + e] = x[e] * scale;
  }
}
// the streamed side's XB_S rows
template <typename IO, int D>
__device__ __forceinline__ void xb_stage(const IO* X, int r0, int n, float scale, float* dst) {
  xb_rows<IO, D, XB_S>(X, r0, n, scale, dst);
}
// the block's XB_T own rows
template <typename IO, int D>
__device__ __forceinline__ void xb_own(const IO* X, int r0, int n, float scale, float* dst) {
  xb_rows<IO, D, XB_T>(X, r0, n, scale, dst);
}

template <int D>
constexpr int xb_lds_bytes() {
  return 4 * (2 * XB_T * (D + 4) + 3 * XB_S * (D + 4) + XB_T * (XB_S + 4) + 2 * XB_S);
}

// grid (ceil(n / 64), BH), block 256.  Online softmax over the keys for the
// block's 64 queries: S (16 x 32 per wave and step) in C layout, o = sum
// exp2(x - m) V accumulated on the matrix cores through an LDS P tile.
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_xstats(XBwdArgs a) {
  extern __shared__ __align__(16) float xb_lds[];
  constexpr int LD = D + 4, CT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, q0 = blockIdx.x * XB_T;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* K = reinterpret_cast<const IO*>(a.k) + (size_t)bh * a.n * D;
  const IO* V = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  float* const Qs = xb_lds;
  float* const Ks = Qs + XB_T * LD;
  float* const Vs = Ks + XB_S * LD;
  float* const Pt = Vs + 2 * XB_S * LD;  // [64][XB_S + 4]
  float* const val = Pt + XB_T * (XB_S + 4);
  xb_own<IO, D>(Q, q0, a.n, a.s4, Qs);
  // per lane: rows 4g + r of the wave's 16 queries (C layout of S), running
  // max and sum over the lane's key columns; o accumulated per (query, channel)
  float mrun[4], lsum[4];
  f32x4 o[CT];  // o[ct][r]: query 4g + r, channel 16 ct + c16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrun[r] = NEG_BIG;
    lsum[r] = 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.n; k0 += XB_S) {
    __syncthreads();
    xb_stage<IO, D>(K, k0, a.n, a.s4, Ks);
    xb_stage<IO, D>(V, k0, a.n, 1.f, Vs);
    if (threadIdx.x < XB_S) {
      const int key = k0 + threadIdx.x;
      val[threadIdx.x] = (key < a.n && (mask == nullptr || mask[key] != 0)) ? 1.f : 0.f;
    }
    __syncthreads();
    f32x4 s[2];
    float tmax[4] = {NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = mm16<D>(Qs + 16 * wave * LD, LD, 1, Ks + 16 * kt * LD, 1, LD, f32x4{0.f, 0.f, 0.f, 0.f});
      const bool ok = val[16 * kt + c16] != 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kt][r] = ok ? s[kt][r] * LOG2E : -INFINITY;
        tmax[r] = fmaxf(tmax[r], s[kt][r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mnew = fmaxf(mrun[r], max16(tmax[r]));
      const float alpha = fast_exp2(mrun[r] - mnew);
      mrun[r] = mnew;
      lsum[r] *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct][r] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float p = fast_exp2(s[kt][r] - mnew);
        lsum[r] += p;
        Pt[(16 * wave + 4 * g + r) * (XB_S + 4) + 16 * kt + c16] = p;
      }
    }
    // o(query, channel) += P V: C(query 4g + r, channel 16 ct + c16) -> keep
    // per lane the r-th query's channel tiles: o[ct][r]
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const f32x4 c = mm16<XB_S>(Pt + 16 * wave * (XB_S + 4), XB_S + 4, 1, Vs + 16 * ct, LD, 1,
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) o[ct][r] += c[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = sum16(lsum[r]);
    const int tok = q0 + 16 * wave + 4 * g + r;
    float dt = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float ov = l > 0.f ? o[ct][r] / l : 0.f;
      const float d = tok < a.n ? io_get(DO + (size_t)tok * D + 16 * ct + c16) : 0.f;
      dt += ov * d;
    }
    dt = sum16(dt);
    if (c16 == 0 && tok < a.n) {
      a.lse[(size_t)bh * a.n + tok] = l > 0.f ? mrun[r] + log2f(l) : INFINITY;
      a.Dt[(size_t)bh * a.n + tok] = dt;
    }
  }
}

// grid (ceil(n / 64), BH), block 256: dq for the block's 64 queries.
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_xq(XBwdArgs a) {
  extern __shared__ __align__(16) float xb_lds[];
  constexpr int LD = D + 4, CT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, q0 = blockIdx.x * XB_T;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* K = reinterpret_cast<const IO*>(a.k) + (size_t)bh * a.n * D;
  const IO* V = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  float* const Qs = xb_lds;
  float* const DOs = Qs + XB_T * LD;
  float* const Ks = DOs + XB_T * LD;
  float* const Vs = Ks + XB_S * LD;
  float* const DS = Vs + 2 * XB_S * LD;  // [64][XB_S + 4]
  float* const val = DS + XB_T * (XB_S + 4);
  xb_own<IO, D>(Q, q0, a.n, a.s4, Qs);
  xb_own<IO, D>(DO, q0, a.n, 1.f, DOs);
  float lse[4], dt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = q0 + 16 * wave + 4 * g + r;
    lse[r] = tok < a.n ? a.lse[(size_t)bh * a.n + tok] : INFINITY;
    dt[r] = tok < a.n ? a.Dt[(size_t)bh * a.n + tok] : 0.f;
  }
  f32x4 dq[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dq[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.n; k0 += XB_S) {
    __syncthreads();
    xb_stage<IO, D>(K, k0, a.n, a.s4, Ks);
    xb_stage<IO, D>(V, k0, a.n, 1.f, Vs);
    if (threadIdx.x < XB_S) {
      const int key = k0 + threadIdx.x;
      val[threadIdx.x] = (key < a.n && (mask == nullptr || mask[key] != 0)) ? 1.f : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const f32x4 s = mm16<D>(Qs + 16 * wave * LD, LD, 1, Ks + 16 * kt * LD, 1, LD,
                               f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 dp = mm16<D>(DOs + 16 * wave * LD, LD, 1, Vs + 16 * kt * LD, 1, LD,
                                f32x4{0.f, 0.f, 0.f, 0.f});
      const bool ok = val[16 * kt + c16] != 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = ok ? exp2f(s[r] * LOG2E - lse[r]) : 0.f;
        DS[(16 * wave + 4 * g + r) * (XB_S + 4) + 16 * kt + c16] = p * (dp[r] - dt[r]);
      }
    }
    // dq += dS Ks (the wave's own 16 rows)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      dq[ct] = mm16<XB_S>(DS + 16 * wave * (XB_S + 4), XB_S + 4, 1, Ks + 16 * ct, LD, 1, dq[ct]);
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = q0 + 16 * wave + 4 * g + r;
      if (tok < a.n) io_put(reinterpret_cast<IO*>(a.dq) + ((size_t)bh * a.n + tok) * D + 16 * ct + c16, a.s4 * dq[ct][r]);
    }
}

// grid (ceil(n / 64), BH), block 256: dk and dv for the block's 64 keys.
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_xkv(XBwdArgs a) {
  extern __shared__ __align__(16) float xb_lds[];
  constexpr int LD = D + 4, CT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, k0 = blockIdx.x * XB_T;
  const IO* Q = reinterpret_cast<const IO*>(a.q) + (size_t)bh * a.n * D;
  const IO* K = reinterpret_cast<const IO*>(a.k) + (size_t)bh * a.n * D;
  const IO* V = reinterpret_cast<const IO*>(a.v) + (size_t)bh * a.n * D;
  const IO* DO = reinterpret_cast<const IO*>(a.dout) + (size_t)bh * a.n * D;
  const uint8_t* mask = a.key_mask ? a.key_mask + (size_t)b * a.n : nullptr;
  float* const Ks = xb_lds;
  float* const Vs = Ks + XB_T * LD;
  float* const Qs = Vs + XB_T * LD;
  float* const DOs = Qs + XB_S * LD;
  float* const Pt = DOs + 2 * XB_S * LD;  // [XB_S queries][64 keys + 4]: P, then dS
  float* const st = Pt + XB_S * (XB_T + 4);   // lse, D of the step's queries
  float* const dst = st + XB_S;
  xb_own<IO, D>(K, k0, a.n, a.s4, Ks);
  xb_own<IO, D>(V, k0, a.n, 1.f, Vs);
  // validity of the wave's own keys (rows of the C tiles below)
  bool ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = k0 + 16 * wave + 4 * g + r;
    ok[r] = key < a.n && (mask == nullptr || mask[key] != 0);
  }
  f32x4 dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < a.n; t0 += XB_S) {
    __syncthreads();
    xb_stage<IO, D>(Q, t0, a.n, a.s4, Qs);
    xb_stage<IO, D>(DO, t0, a.n, 1.f, DOs);
    if (threadIdx.x < XB_S) {
      const int tok = t0 + threadIdx.x;
      st[threadIdx.x] = tok < a.n ? a.lse[(size_t)bh * a.n + tok] : INFINITY;
      dst[threadIdx.x] = tok < a.n ? a.Dt[(size_t)bh * a.n + tok] : 0.f;
    }
    __syncthreads();
    // S^T (keys x queries): C(key 4g + r of the wave's 16, query 16 qt + c16)
    f32x4 p[2], ds[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const f32x4 s = mm16<D>(Ks + 16 * wave * LD, LD, 1, Qs + 16 * qt * LD, 1, LD,
                               f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 dp = mm16<D>(Vs + 16 * wave * LD, LD, 1, DOs + 16 * qt * LD, 1, LD,
                                f32x4{0.f, 0.f, 0.f, 0.f});
      const int qq = 16 * qt + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[qt][r] = ok[r] ? exp2f(s[r] * LOG2E - st[qq]) : 0.f;
        ds[qt][r] = p[qt][r] * (dp[r] - dst[qq]);
      }
    }
    // dv += P^T dout, dk += dS^T Qs over the step's 32 queries: the wave's own
    // 16 keys as rows; P^T / dS^T go through the wave's own LDS columns
    float* const myP = Pt;  // [query][key]: column 16 wave + 4 g + r
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          myP[(16 * qt + c16) * (XB_T + 4) + 16 * wave + 4 * g + r] = pass == 0 ? p[qt][r] : ds[qt][r];
      // A(key i, query k) = myP[k][16 wave + i]
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (pass == 0)
          dv[ct] = mm16<XB_S>(myP + 16 * wave, 1, XB_T + 4, DOs + 16 * ct, LD, 1, dv[ct]);
        else
          dk[ct] = mm16<XB_S>(myP + 16 * wave, 1, XB_T + 4, Qs + 16 * ct, LD, 1, dk[ct]);
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 16 * wave + 4 * g + r;
      if (key >= a.n) continue;
      const size_t o = ((size_t)bh * a.n + key) * D + 16 * ct + c16;
      io_put(reinterpret_cast<IO*>(a.dv) + o, dv[ct][r] + (a.dvc != nullptr ? a.dvc[o] : 0.f));
      io_put(reinterpret_cast<IO*>(a.dk) + o, a.s4 * dk[ct][r]);
    }
}

}  // namespace nys
