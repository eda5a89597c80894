// Iterative Moore-Penrose inverse of the landmark kernel A.
//
// Page: "Nystromformer 源码解析与实战指南" (blog.gitcode.com), section 2.5:
// Z_0 = A^T / c, then n_iter times X = A Z and
// Z <- (1/4) Z (13 I - X (15 I - X (7 I - X))).  The init scale c is
// (max column sum) * (max row sum) of A, taken over every head of the call
// for the default ("original") option and per head for the exact-coefficient
// option.
//
// The iteration is kept literally (X is recomputed from A and Z every step),
// which is what keeps it self-correcting in finite precision.  Products are
// split-bf16 matrix-core products (hi*hi + hi*lo + lo*hi, float32-accurate).
//
// pinv_block<M> (M <= 128): one workgroup per head, everything on chip.
//   Wave w owns the 16-row tiles {w, w+4} of A, X and Z and keeps them in
//   registers as operand fragments.  The matrices every wave needs whole
//   (Z as a right factor, 7I - X, 15I - T1, 13I - T2) pass through two LDS
//   regions R0 / R1 in column-major bf16 hi/lo form: each step reads one
//   region and writes the other, so two M x M buffers suffice (M = 128 fits
//   the 160 KB LDS).  Steps 1 and 4 are computed transposed
//   (X^T = Z^T A^T, Z'^T = (13I - T2)^T Z^T /4) so that their C tiles land in
//   each lane as the row fragments the next products need (paired k order).
//
// k_pinv_init / k_pinv_gemm (M > 128): the same iteration as a sequence of
//   batched launches, one product per launch, with the matrices in global
//   memory; the kernel boundaries are the step barriers.
#pragma once

#include "common.hpp"

namespace nys {

struct PinvArgs {
  const float* A;       // [BH][M][M]
  const float* colmax;  // [BH]
  const float* rowmax;  // [BH]
  float* Z;             // [BH][M][M] out
  float* cscale;        // [BH] out
  int BH, n_iter, init_option;
};

__device__ __forceinline__ float pinv_scale(const PinvArgs& a, int bh) {
  if (a.init_option == 0) {
    float cm = 0.f, rm = 0.f;
    for (int i = threadIdx.x & 63; i < a.BH; i += 64) {
      cm = fmaxf(cm, a.colmax[i]);
      rm = fmaxf(rm, a.rowmax[i]);
    }
    cm = wave_max(cm);
    rm = wave_max(rm);
    return cm * rm;
  }
  return a.colmax[bh] * a.rowmax[bh];
}

template <int M>
constexpr int pinv_lds_bytes() {
  return 4 * M * (M + 8) * 2;  // two regions, hi + lo, bf16
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int M>
__device__ void pinv_block(const PinvArgs& a, int bh, __bf16* lds) {
  constexpr int TM = M / 16, KS = M / 32, LD = M + 8;
  constexpr int OWN = (TM + 3) / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  __bf16* const R0h = lds;
  __bf16* const R0l = lds + M * LD;
  __bf16* const R1h = lds + 2 * M * LD;
  __bf16* const R1l = lds + 3 * M * LD;
  const float* A = a.A + (size_t)bh * M * M;
  float* Zg = a.Z + (size_t)bh * M * M;

  const float c = pinv_scale(a, bh);
  const float invc = 1.0f / c;
  if (threadIdx.x == 0) a.cscale[bh] = c;
  if (a.n_iter == 0) {
    for (int idx = threadIdx.x; idx < M * M; idx += 256) {
      const int row = idx / M, col = idx % M;
      Zg[idx] = A[(size_t)col * M + row] * invc;
    }
    return;
  }

  Frag2 Af[OWN][KS], Xf[OWN][KS], Zf[OWN][KS];
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int t = wave + 4 * o;
    if (t < TM) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = A[(size_t)(16 * t + c16) * M + 32 * ks + 8 * g + e];
        Af[o][ks] = split8(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kp = 32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
          x[e] = A[(size_t)kp * M + 16 * t + c16] * invc;
        }
        Zf[o][ks] = split8(x);
      }
    }
  }
  // R0 <- Z_0 column-major: element (row, col) at col * LD + row
  for (int idx = threadIdx.x; idx < M * M; idx += 256) {
    const int col = idx / M, row = idx % M;
    __bf16 h, l;
    split1(A[(size_t)col * M + row] * invc, h, l);
    R0h[col * LD + row] = h;
    R0l[col * LD + row] = l;
  }
  __syncthreads();

  for (int it = 0; it < a.n_iter; ++it) {
    const bool last = (it == a.n_iter - 1);
    // ---- step 1: X^T[:, t] = Z^T A^T[:, t]; keep X rows, store 7I - X in R1
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int t = wave + 4 * o;
      if (t >= TM) continue;
      f32x4 acc[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag2 zt;
          zt.hi = *reinterpret_cast<const bf16x8*>(R0h + (16 * i + c16) * LD + 32 * ks + 8 * g);
          zt.lo = *reinterpret_cast<const bf16x8*>(R0l + (16 * i + c16) * LD + 32 * ks + 8 * g);
          acc[i] = mma<3>(zt, Af[o][ks], acc[i]);
        }
      }
      // acc[i][r] = X[16t + c16][16i + 4g + r]
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8] = {acc[2 * ks][0], acc[2 * ks][1], acc[2 * ks][2], acc[2 * ks][3],
                      acc[2 * ks + 1][0], acc[2 * ks + 1][1], acc[2 * ks + 1][2], acc[2 * ks + 1][3]};
        Xf[o][ks] = split8(x);
      }
      const int row = 16 * t + c16;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = 16 * i + 4 * g + r;
          __bf16 h, l;
          split1((row == col ? 7.f : 0.f) - acc[i][r], h, l);
          R1h[col * LD + row] = h;
          R1l[col * LD + row] = l;
        }
    }
    __syncthreads();
    // ---- steps 2 and 3: T = X (diag - prev); store (next diag - T) column-major
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const __bf16* Bh = step == 0 ? R1h : R0h;
      const __bf16* Bl = step == 0 ? R1l : R0l;
      __bf16* Oh = step == 0 ? R0h : R1h;
      __bf16* Ol = step == 0 ? R0l : R1l;
      const float diag = step == 0 ? 15.f : 13.f;
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int t = wave + 4 * o;
        if (t >= TM) continue;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          const int col = 16 * j + c16;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int k0 = col * LD + 32 * ks + 4 * g;
            Frag2 bfr;
            bfr.hi = cat44(*reinterpret_cast<const bf16x4*>(Bh + k0), *reinterpret_cast<const bf16x4*>(Bh + k0 + 16));
            bfr.lo = cat44(*reinterpret_cast<const bf16x4*>(Bl + k0), *reinterpret_cast<const bf16x4*>(Bl + k0 + 16));
            acc = mma<3>(Xf[o][ks], bfr, acc);
          }
          // acc[r] = T[16t + 4g + r][col]
          bf16x4 h4, l4;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * t + 4 * g + r;
            __bf16 h, l;
            split1((row == col ? diag : 0.f) - acc[r], h, l);
            h4[r] = h;
            l4[r] = l;
          }
          *reinterpret_cast<bf16x4*>(Oh + col * LD + 16 * t + 4 * g) = h4;
          *reinterpret_cast<bf16x4*>(Ol + col * LD + 16 * t + 4 * g) = l4;
        }
      }
      __syncthreads();
    }
    // ---- step 4: Z'^T[:, t] = (13I - T2)^T Z^T[:, t] / 4 (R1 holds 13I - T2)
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int t = wave + 4 * o;
      if (t >= TM) continue;
      f32x4 acc[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int k0 = (16 * i + c16) * LD + 32 * ks + 4 * g;
          Frag2 afr;
          afr.hi = cat44(*reinterpret_cast<const bf16x4*>(R1h + k0), *reinterpret_cast<const bf16x4*>(R1h + k0 + 16));
          afr.lo = cat44(*reinterpret_cast<const bf16x4*>(R1l + k0), *reinterpret_cast<const bf16x4*>(R1l + k0 + 16));
          acc[i] = mma<3>(afr, Zf[o][ks], acc[i]);
        }
        acc[i] *= 0.25f;
      }
      // acc[i][r] = Z'[16t + c16][16i + 4g + r]
      const int row = 16 * t + c16;
      if (last) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          *reinterpret_cast<float4*>(Zg + (size_t)row * M + 16 * i + 4 * g) =
              make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float x[8] = {acc[2 * ks][0], acc[2 * ks][1], acc[2 * ks][2], acc[2 * ks][3],
                        acc[2 * ks + 1][0], acc[2 * ks + 1][1], acc[2 * ks + 1][2], acc[2 * ks + 1][3]};
          Zf[o][ks] = split8(x);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = 16 * i + 4 * g + r;
            __bf16 h, l;
            split1(acc[i][r], h, l);
            R0h[col * LD + row] = h;
            R0l[col * LD + row] = l;
          }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// M > 128: the iteration as a launch sequence over global memory.

// grid: BH blocks of 256: c, then Z = A^T / c.
__global__ __launch_bounds__(256) void k_pinv_init(PinvArgs a, int M) {
  const int bh = blockIdx.x;
  const float c = pinv_scale(a, bh);
  const float invc = 1.0f / c;
  if (threadIdx.x == 0) a.cscale[bh] = c;
  const float* A = a.A + (size_t)bh * M * M;
  float* Z = a.Z + (size_t)bh * M * M;
  for (int idx = threadIdx.x; idx < M * M; idx += 256) {
    const int row = idx / M, col = idx % M;
    Z[idx] = A[(size_t)col * M + row] * invc;
  }
}

// C = alpha * P * Q' with Q' = Q when beta == 0, else beta * I - Q.
// grid: ((M/32)^2, BH), block 256 (4 waves, one 16x16 tile each).
__global__ __launch_bounds__(256) void k_pinv_gemm(const float* __restrict__ P, const float* __restrict__ Q,
                                                    float* __restrict__ C, int M, float beta, float alpha) {
  const int bh = blockIdx.y;
  const int nb = M / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int row0 = (blockIdx.x / nb) * 32 + (wave >> 1) * 16;
  const int col0 = (blockIdx.x % nb) * 32 + (wave & 1) * 16;
  const float* Pm = P + (size_t)bh * M * M;
  const float* Qm = Q + (size_t)bh * M * M;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < M / 32; ++ks) {
    float x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 32 * ks + 8 * g + e;
      x[e] = Pm[(size_t)(row0 + c16) * M + k];
      const float qv = Qm[(size_t)k * M + col0 + c16];
      y[e] = beta != 0.f ? ((k == col0 + c16 ? beta : 0.f) - qv) : qv;
    }
    acc = mma<3>(split8(x), split8(y), acc);
  }
  float* Cm = C + (size_t)bh * M * M;
#pragma unroll
  for (int r = 0; r < 4; ++r) Cm[(size_t)(row0 + 4 * g + r) * M + col0 + c16] = alpha * acc[r];
}

}  // namespace nys
