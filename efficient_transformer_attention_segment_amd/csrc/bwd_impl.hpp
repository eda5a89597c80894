// Backward launch sequences (Nystrom path and exact branch), shared by
// bwd_f32.hip and bwd_bf16.hip, each of which instantiates run_backward for
// its I/O type.  The forward stages the backward recomputes come from the
// forward units (dispatch_m with the plan's bwd flag set).
#pragma once

#include <cmath>

#include "host.hpp"
#include "k_bwd.hpp"

namespace nys {
namespace host {

// ------------------------------------------------------------ backward ---
// Forward stages (without the output pass) into the plan's workspace, then
// the backward kernels into the regions that follow it.
struct BwdPlan {
  int nct, nck, ncv, mats;
  size_t off_dqf, off_pw, off_pk, off_pq, off_mm, off_dW, off_dBV, off_dQt, off_dKt, off_Dv, off_dc, off_cmax,
      off_cmaxj, off_rmax, off_dvc, off_pconv, off_dvk, total;
};

inline BwdPlan make_bwd_plan(const Plan& p, int n_iter, int conv_k, bool conv) {
  BwdPlan b{};
  const int ct = bwd_tok_chunk(p.m, p.D);
  b.nct = (p.n + ct - 1) / ct;
  const int ck = bwd_key_chunk(p.m, p.D);
  b.nck = (p.n + ck - 1) / ck;
  b.ncv = (p.n + BWD_CV - 1) / BWD_CV;
  b.mats = bwd_mm_mats(n_iter);
  const size_t BH = p.BH, M = p.m, n = p.n, D = p.D;
  size_t o = p.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  b.off_dqf = take(BH * n * D * 4);
  b.off_pw = take(BH * b.nct * M * D * 4);
  b.off_pk = take(BH * b.nct * M * D * 4);
  b.off_pq = take(BH * b.nck * M * D * 4);
  b.off_mm = take(BH * b.mats * M * M * 4);
  b.off_dW = take(BH * M * D * 4);
  b.off_dBV = take(BH * M * D * 4);
  b.off_dQt = take(BH * M * D * 4);
  b.off_dKt = take(BH * M * D * 4);
  b.off_Dv = take(BH * M * 4);
  b.off_dc = take(BH * 4);
  b.off_cmax = take(BH * 4);
  b.off_cmaxj = take(BH * 4);
  b.off_rmax = take(BH * 4);
  b.off_dvc = conv ? take(BH * n * D * 4) : 0;
  b.off_pconv = conv ? take(BH * b.ncv * (size_t)conv_k * 4) : 0;
  b.off_dvk = M > 128 ? take(2 * BH * n * D * 4) : 0;  // the key pass's first-half dv, dk
  b.total = o;
  return b;
}

// The pseudo-inverse backward above 64 landmarks as a launch chain
// (k_bwd_chain, every head per launch).  Forward half (it needs only A and
// c, so it runs beside the token pass): Z_0, then per iteration X_k = A Z_k,
// X_k^2, P_k and Z_k+1 (all kept).  Backward half: dW and dKt from the token
// partials, dZ_n = dW BV^T with dBV = Z_n^T dW, then per iteration, last
// first, with G the gradient reaching Z_k+1:
//   dZ_k = G P^T / 4 and dP = Z^T G / 4;
//   T = X^T dP and dX = 7 dP X^T + 7 X^T dP - dP (X^2)^T - (X^2)^T dP - 15 dP;
//   dX -= T X^T;
//   dA += dX Z^T and dZ_k += A^T dX;
// and the end (k_bwd_chain_post, k_bwd_chain_dc; A's statistics come from
// k_bwd_chain_stats in the forward half).  The same products and scratch layout as
// k_bwd_mm1 (the matrices of a head at a.mm + h * bwd_mm_mats(n_iter) M^2).
template <int M, int D>
struct BwdChain {
  static constexpr int KMAX = M > D ? M : D;
  static constexpr long long MM = (long long)M * M, MD = (long long)M * D;
  const Plan& p;
  const BwdArgs& a;
  int n_iter;
  long long sm;  // per-head stride of the scratch matrices
  BwdChain(const Plan& p_, const BwdArgs& a_, int n) : p(p_), a(a_), n_iter(n), sm((long long)bwd_mm_mats(n) * MM) {}
  float* Z(int k) const { return a.mm + k * MM; }
  float* X(int k) const { return a.mm + (n_iter + 1 + 3 * k) * MM; }
  float* X2(int k) const { return X(k) + MM; }
  float* P(int k) const { return X(k) + 2 * MM; }
  float* G() const { return a.mm + (4 * n_iter + 1) * MM; }
  // op(x) is R x K and op(y) is K x N
  static ChainTerm term(const float* x, long long sx, bool tx, const float* y, long long sy, bool ty, float alpha,
                        const ChainOut& o) {
    ChainTerm t{};
    t.a = x;
    t.b = y;
    t.sa = sx;
    t.sb = sy;
    t.ta = tx;
    t.tb = ty;
    t.lda = tx ? o.R : o.K;
    t.ldb = ty ? o.K : o.N;
    t.alpha = alpha;
    return t;
  }
  static ChainOut out(float* c, long long sc, int R, int N, int K, float beta) {
    ChainOut o{};
    o.c = c;
    o.sc = sc;
    o.R = R;
    o.N = N;
    o.K = K;
    o.ldc = N;
    o.beta = beta;
    return o;
  }
  hipError_t go(const ChainOut& o0, const ChainOut* o1, hipStream_t st) const {
    ChainLaunch L{};
    L.o[0] = o0;
    L.tiles0 = chain_tiles(o0.R, o0.N);
    int tiles = L.tiles0;
    if (o1 != nullptr) {
      L.o[1] = *o1;
      tiles += chain_tiles(o1->R, o1->N);
    }
    return launch("k_bwd_chain", k_bwd_chain<KMAX>, dim3(tiles, p.BH), dim3(256), (uint32_t)chain_lds_bytes<KMAX>(),
                  st, L);
  }
  int forward(hipStream_t st) const {
    HIP_TRY(launch("k_bwd_chain_init", k_bwd_chain_init<M>, dim3((unsigned)((MM + 255) / 256), p.BH), dim3(256), 0,
                   st, a));
    HIP_TRY(launch("k_bwd_chain_stats", k_bwd_chain_stats<M>, dim3(p.BH), dim3(BWD_MM_NT), 0, st, a));
    HIP_TRY(allow_lds(k_bwd_chain<KMAX>, chain_lds_bytes<KMAX>()));
    for (int k = 0; k < n_iter; ++k) {
      ChainOut o = out(X(k), sm, M, M, M, 0.f);  // X = A Z
      o.t[o.nt++] = term(a.A, MM, false, Z(k), sm, false, 1.f, o);
      HIP_TRY(go(o, nullptr, st));
      o = out(X2(k), sm, M, M, M, 0.f);  // X^2
      o.t[o.nt++] = term(X(k), sm, false, X(k), sm, false, 1.f, o);
      HIP_TRY(go(o, nullptr, st));
      o = out(P(k), sm, M, M, M, 0.f);  // P = 13I - 15X + 7X^2 - X^3
      o.t[o.nt++] = term(X(k), sm, false, X2(k), sm, false, -1.f, o);
      o.e1 = X(k);
      o.g1 = -15.f;
      o.e2 = X2(k);
      o.g2 = 7.f;
      o.eye = 13.f;
      HIP_TRY(go(o, nullptr, st));
      o = out(Z(k + 1), sm, M, M, M, 0.f);  // Z <- Z P / 4
      o.t[o.nt++] = term(Z(k), sm, false, P(k), sm, false, 0.25f, o);
      HIP_TRY(go(o, nullptr, st));
    }
    return NYS_OK;
  }
  // after the token pass on st; the forward half joins through fwd_done
  int backward(hipStream_t st, hipEvent_t fwd_done) const {
    static_assert(M * D % 4 == 0, "four-element groups");
    HIP_TRY(launch("k_bwd_chain_sum", k_bwd_chain_sum<M, D>, dim3((unsigned)((MD + 255) / 256), p.BH), dim3(256), 0,
                   st, a));
    if (fwd_done != nullptr) HIP_TRY(hipStreamWaitEvent(st, fwd_done, 0));
    float* const Gm = G();
    float* const Gn = Gm + MM;
    float* const dP = Gm + 2 * MM;
    float* const dX = Gm + 3 * MM;
    float* const T = Gm + 4 * MM;
    float* const dA = Gm + 5 * MM;
    {
      ChainOut o0 = out(Gm, sm, M, M, D, 0.f);  // dZ_n = dW BV^T
      o0.t[o0.nt++] = term(a.dW, MD, false, a.BV, MD, true, 1.f, o0);
      ChainOut o1 = out(a.dBV, MD, M, D, M, 0.f);  // dBV = Z_n^T dW
      o1.t[o1.nt++] = term(Z(n_iter), sm, true, a.dW, MD, false, 1.f, o1);
      HIP_TRY(go(o0, &o1, st));
    }
    float* g = Gm;
    float* gn = Gn;
    for (int k = n_iter - 1; k >= 0; --k) {
      ChainOut o0 = out(gn, sm, M, M, M, 0.f);
      o0.t[o0.nt++] = term(g, sm, false, P(k), sm, true, 0.25f, o0);
      ChainOut o1 = out(dP, sm, M, M, M, 0.f);
      o1.t[o1.nt++] = term(Z(k), sm, true, g, sm, false, 0.25f, o1);
      HIP_TRY(go(o0, &o1, st));
      o0 = out(T, sm, M, M, M, 0.f);
      o0.t[o0.nt++] = term(X(k), sm, true, dP, sm, false, 1.f, o0);
      o1 = out(dX, sm, M, M, M, 0.f);
      o1.t[o1.nt++] = term(dP, sm, false, X(k), sm, true, 7.f, o1);
      o1.t[o1.nt++] = term(X(k), sm, true, dP, sm, false, 7.f, o1);
      o1.t[o1.nt++] = term(dP, sm, false, X2(k), sm, true, -1.f, o1);
      o1.t[o1.nt++] = term(X2(k), sm, true, dP, sm, false, -1.f, o1);
      o1.e1 = dP;
      o1.g1 = -15.f;
      HIP_TRY(go(o0, &o1, st));
      o0 = out(dX, sm, M, M, M, 1.f);
      o0.t[o0.nt++] = term(T, sm, false, X(k), sm, true, -1.f, o0);
      HIP_TRY(go(o0, nullptr, st));
      o0 = out(dA, sm, M, M, M, 1.f);
      o0.t[o0.nt++] = term(dX, sm, false, Z(k), sm, true, 1.f, o0);
      o1 = out(gn, sm, M, M, M, 1.f);
      o1.t[o1.nt++] = term(a.A, MM, true, dX, sm, false, 1.f, o1);
      HIP_TRY(go(o0, &o1, st));
      float* const t = g;
      g = gn;
      gn = t;
    }
    const int gsel = 4 * n_iter + 1 + (g == Gm ? 0 : 1);
    HIP_TRY(launch("k_bwd_chain_post", k_bwd_chain_post<M>, dim3((M / 32) * (M / 32), p.BH), dim3(256), 0, st, a,
                   gsel));
    HIP_TRY(launch("k_bwd_chain_dc", k_bwd_chain_dc<M>, dim3(p.BH), dim3(64), 0, st, a));
    return NYS_OK;
  }
  // after k_bwd_mm2<M, D, true> (dS_A in the T slot): dQt_A = dS_A Kt and
  // dKt += dS_A^T Qt
  int mm2_products(hipStream_t st) const {
    const float* const dSA = G() + 4 * MM;
    ChainOut o0 = out(a.dQt, MD, M, D, M, 0.f);
    o0.t[o0.nt++] = term(dSA, sm, false, a.kt, MD, false, 1.f, o0);
    ChainOut o1 = out(a.dKt, MD, M, D, M, 1.f);
    o1.t[o1.nt++] = term(dSA, sm, true, a.qt, MD, false, 1.f, o1);
    HIP_TRY(go(o0, &o1, st));
    return NYS_OK;
  }
};

template <typename IO, int M, int D>
int launch_backward(const Plan& p, const BwdPlan& bp, Workspace* w, const void* q, const void* k, const void* v,
                    const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option,
                    const void* dout, void* dq, void* dk, void* dv, float* dconv_w, hipStream_t st) {
  int rc = dispatch_m<IO, D>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, nullptr, st);
  if (rc != NYS_OK) return rc;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.key_mask = mask;
  a.conv_w = conv_w;
  a.conv_k = conv_k;
  a.qt = at<float>(w, p.off_qt);
  a.kt = at<float>(w, p.off_kt);
  a.A = at<float>(w, p.off_A);
  a.BV = at<float>(w, p.off_BV);
  a.W = at<float>(w, p.off_W);
  a.lse = at<float>(w, p.off_lse);
  a.cscale = at<float>(w, p.off_cscale);
  a.dqf = at<float>(w, bp.off_dqf);
  a.pw = at<float>(w, bp.off_pw);
  a.pk = at<float>(w, bp.off_pk);
  a.pq = at<float>(w, bp.off_pq);
  a.mm = at<float>(w, bp.off_mm);
  a.dW = at<float>(w, bp.off_dW);
  a.dBV = at<float>(w, bp.off_dBV);
  a.dQt = at<float>(w, bp.off_dQt);
  a.dKt = at<float>(w, bp.off_dKt);
  a.Dv = at<float>(w, bp.off_Dv);
  a.dc = at<float>(w, bp.off_dc);
  a.cmax = at<float>(w, bp.off_cmax);
  a.cmaxj = at<int>(w, bp.off_cmaxj);
  a.rmax = at<float>(w, bp.off_rmax);
  a.dvc = conv_w != nullptr ? at<float>(w, bp.off_dvc) : nullptr;
  a.pconv = conv_w != nullptr ? at<float>(w, bp.off_pconv) : nullptr;
  a.dvk = M > 128 ? at<float>(w, bp.off_dvk) : nullptr;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dconv_w = dconv_w;
  a.n = p.n;
  a.H = p.H;
  a.BH = p.BH;
  a.mr = p.mr;
  a.L = p.L;
  a.nct = bp.nct;
  a.nck = bp.nck;
  a.ncv = bp.ncv;
  a.n_iter = n_iter;
  a.init_option = init_option;
  a.s4 = 1.0f / sqrtf(sqrtf((float)D));
  // Side stream: the forward half of the pseudo-inverse backward (it needs
  // only A and c: one workgroup per head at 64 landmarks, the launch chain
  // above) runs beside the token pass; then the conv's backward (it needs
  // only dout, v and the weights, and ends with dconv_w) runs beside the
  // rest of the chain.  Both join back before the kernels that read their
  // results.
  constexpr bool SPLIT = M == 64, CHAIN = M > 64;
  const BwdChain<M, D> chain(p, a, n_iter);
  Side* sd = nullptr;
  if (SPLIT || CHAIN || conv_w != nullptr) {
    rc = get_side(&sd);
    if (rc != NYS_OK) return rc;
    HIP_TRY(hipEventRecord(sd->fork, st));
    HIP_TRY(hipStreamWaitEvent(sd->st, sd->fork, 0));
  }
  if constexpr (SPLIT) {
    HIP_TRY(allow_lds(k_bwd_mm1f64, BWD_MM64_LDS));
    HIP_TRY(launch("k_bwd_mm1f", k_bwd_mm1f64, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)BWD_MM64_LDS, sd->st, a));
    HIP_TRY(hipEventRecord(sd->mid, sd->st));
  }
  if constexpr (CHAIN) {
    rc = chain.forward(sd->st);
    if (rc != NYS_OK) return rc;
    HIP_TRY(hipEventRecord(sd->mid, sd->st));
  }
  if constexpr (bwd_tok2(M, D)) {
    constexpr int tl = BwdTok2Layout<IO, M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_tok2<IO, M, D>, tl));
    HIP_TRY(launch("k_bwd_tok", k_bwd_tok2<IO, M, D>, dim3(bp.nct, p.BH), dim3(256), (uint32_t)tl, st, a));
  } else if constexpr (bwd_tok3(M, D)) {
    constexpr int tl = BwdTok3Layout<M>::BYTES;
    HIP_TRY(allow_lds(k_bwd_tok3<IO, M>, tl));
    HIP_TRY(launch("k_bwd_tok", k_bwd_tok3<IO, M>, dim3(bp.nct, p.BH), dim3(64 * BwdTok3Layout<M>::NW), (uint32_t)tl,
                   st, a));
  } else {
    constexpr int tl = BwdTokLayout<M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_tok<IO, M, D>, tl));
    HIP_TRY(launch("k_bwd_tok", k_bwd_tok<IO, M, D>, dim3(bp.nct, p.BH, BwdTokLayout<M, D>::SPLIT),
                   dim3(64 * bwd_tok_waves<M>()), (uint32_t)tl, st, a));
  }
  if (conv_w != nullptr) {
    HIP_TRY(hipEventRecord(sd->done, st));  // token pass done
    HIP_TRY(hipStreamWaitEvent(sd->st, sd->done, 0));
    constexpr int dl = bwd_dv_lds<D>(), cl = bwd_cv_lds<D>();
    HIP_TRY(allow_lds(k_bwd_dvconv<IO, D>, dl));
    HIP_TRY(launch("k_bwd_dvconv", k_bwd_dvconv<IO, D>, dim3((p.n + BWD_DV_TOK - 1) / BWD_DV_TOK, p.BH), dim3(256),
                   (uint32_t)dl, sd->st, a));
    if (dconv_w != nullptr) {
      HIP_TRY(allow_lds(k_bwd_conv<IO, D>, cl));
      HIP_TRY(launch("k_bwd_conv", k_bwd_conv<IO, D>, dim3(bp.ncv, p.BH), dim3(256), (uint32_t)cl, sd->st, a));
      HIP_TRY(launch("k_bwd_wsum", k_bwd_wsum, dim3(p.H), dim3(1024), 0, sd->st, a));
    }
    HIP_TRY(hipEventRecord(sd->join, sd->st));
  }
  constexpr int ml = bwd_mm_lds_bytes<M, D>();
  if constexpr (SPLIT) {
    HIP_TRY(hipStreamWaitEvent(st, sd->mid, 0));
    if constexpr (sizeof(IO) == 4) {
      HIP_TRY(allow_lds(k_bwd_mm1b64_f32<D>, BWD_MM64B_LDS));
      HIP_TRY(launch("k_bwd_mm1", k_bwd_mm1b64_f32<D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)BWD_MM64B_LDS, st, a));
    } else {
      HIP_TRY(allow_lds(k_bwd_mm1b64<D>, BWD_MM1B_LDS));
      HIP_TRY(launch("k_bwd_mm1", k_bwd_mm1b64<D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)BWD_MM1B_LDS, st, a));
    }
  } else if constexpr (CHAIN) {
    rc = chain.backward(st, sd->mid);
    if (rc != NYS_OK) return rc;
  } else {
    HIP_TRY(allow_lds(k_bwd_mm1<M, D>, ml));
    HIP_TRY(launch("k_bwd_mm1", k_bwd_mm1<M, D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)ml, st, a));
  }
  if constexpr (CHAIN) {
    HIP_TRY(launch("k_bwd_mm2", k_bwd_mm2<M, D, true>, dim3(p.BH), dim3(BWD_MM_NT), 0, st, a));
    rc = chain.mm2_products(st);
    if (rc != NYS_OK) return rc;
  } else {
    HIP_TRY(allow_lds(k_bwd_mm2<M, D>, ml));
    HIP_TRY(launch("k_bwd_mm2", k_bwd_mm2<M, D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)ml, st, a));
  }
  if (conv_w != nullptr) HIP_TRY(hipStreamWaitEvent(st, sd->join, 0));
  if constexpr (bwd_tok2(M, D)) {
    constexpr int kl = BwdKey2Layout<IO, M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_key2<IO, M, D>, kl));
    HIP_TRY(launch("k_bwd_key", k_bwd_key2<IO, M, D>, dim3(bp.nck, p.BH), dim3(256), (uint32_t)kl, st, a));
  } else {
    constexpr int kl = BwdKeyLayout<M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_key<IO, M, D>, kl));
    HIP_TRY(launch("k_bwd_key", k_bwd_key<IO, M, D>, dim3(bp.nck, p.BH), dim3(BWD_KEY_NT), (uint32_t)kl, st, a));
  }
  static_assert((M * D) % 256 == 0, "k_bwd_qt: one element per thread");
  HIP_TRY(launch("k_bwd_qt", k_bwd_qt<M, D>, dim3(M * D / 256, p.BH), dim3(256), 0, st, a));
  HIP_TRY(launch("k_bwd_q", k_bwd_q<IO, M, D>, dim3((p.n + 63) / 64, p.BH), dim3(256), 0, st, a));
  return NYS_OK;
}

// Exact branch (m == n): the conv backward, then the three flash-style passes.
template <typename IO, int D>
int launch_backward_exact(int B, int H, int n, const void* q, const void* k, const void* v, const uint8_t* mask,
                          const float* conv_w, int conv_k, const void* dout, void* dq, void* dk, void* dv,
                          float* dconv_w, hipStream_t st) {
  const size_t BH = (size_t)B * H;
  const int ncv = (n + BWD_CV - 1) / BWD_CV;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  take(HEAD_BYTES);  // zero page and status word, as in every workspace
  const size_t off_lse = take(BH * n * 4), off_dt = take(BH * n * 4);
  const size_t off_dvc = conv_w ? take(BH * n * D * 4) : 0, off_pconv = conv_w ? take(BH * ncv * conv_k * 4) : 0;
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace* w = nullptr;
  int rc = get_workspace(st, o, &w);
  if (rc != NYS_OK) return rc;
  BwdArgs c{};
  c.v = v;
  c.dout = dout;
  c.conv_w = conv_w;
  c.conv_k = conv_k;
  c.dvc = conv_w ? at<float>(w, off_dvc) : nullptr;
  c.pconv = conv_w ? at<float>(w, off_pconv) : nullptr;
  c.dconv_w = dconv_w;
  c.n = n;
  c.H = H;
  c.BH = (int)BH;
  c.ncv = ncv;
  if (conv_w != nullptr) {
    constexpr int dl = bwd_dv_lds<D>(), cl = bwd_cv_lds<D>();
    HIP_TRY(allow_lds(k_bwd_dvconv<IO, D>, dl));
    HIP_TRY(launch("k_bwd_dvconv", k_bwd_dvconv<IO, D>, dim3((n + BWD_DV_TOK - 1) / BWD_DV_TOK, (unsigned)BH),
                   dim3(256), (uint32_t)dl, st, c));
    if (dconv_w != nullptr) {
      HIP_TRY(allow_lds(k_bwd_conv<IO, D>, cl));
      HIP_TRY(launch("k_bwd_conv", k_bwd_conv<IO, D>, dim3(ncv, (unsigned)BH), dim3(256), (uint32_t)cl, st, c));
    }
  }
  XBwdArgs x{};
  x.q = q;
  x.k = k;
  x.v = v;
  x.dout = dout;
  x.key_mask = mask;
  x.dvc = c.dvc;
  x.lse = at<float>(w, off_lse);
  x.Dt = at<float>(w, off_dt);
  x.dq = dq;
  x.dk = dk;
  x.dv = dv;
  x.n = n;
  x.H = H;
  x.s4 = 1.0f / sqrtf(sqrtf((float)D));
  const dim3 grid((n + XB_T - 1) / XB_T, (unsigned)BH);
  constexpr int xl = xb_lds_bytes<D>();
  HIP_TRY(allow_lds(k_bwd_xstats<IO, D>, xl));
  HIP_TRY(launch("k_bwd_xstats", k_bwd_xstats<IO, D>, grid, dim3(256), (uint32_t)xl, st, x));
  HIP_TRY(allow_lds(k_bwd_xq<IO, D>, xl));
  HIP_TRY(launch("k_bwd_xq", k_bwd_xq<IO, D>, grid, dim3(256), (uint32_t)xl, st, x));
  HIP_TRY(allow_lds(k_bwd_xkv<IO, D>, xl));
  HIP_TRY(launch("k_bwd_xkv", k_bwd_xkv<IO, D>, grid, dim3(256), (uint32_t)xl, st, x));
  if (conv_w != nullptr && dconv_w != nullptr)
    HIP_TRY(launch("k_bwd_wsum", k_bwd_wsum, dim3(H), dim3(1024), 0, st, c));
  return NYS_OK;
}

template <typename IO>
int run_backward(const void* q, const void* k, const void* v, const uint8_t* mask, const float* conv_w, int conv_k,
                 int B, int H, int n, int d, int m, int n_iter, int init_option, const void* dout, void* dq, void* dk,
                 void* dv, float* dconv_w, hipStream_t st) {
  int rc = validate(sizeof(IO), q, k, v, B, H, n, d, m, n_iter, init_option, dq);
  if (rc != NYS_OK) return rc;
  if (!dout || !dk || !dv) return fail(NYS_ERR_INVALID, "dout, dq, dk and dv must be non-NULL");
  if (conv_w != nullptr) {
    if (conv_k < 1 || conv_k % 2 == 0)
      return fail(NYS_ERR_INVALID, "conv_kernel_size=%d: 'same' padding needs an odd size >= 1", conv_k);
    if (conv_k > TAPS) return fail(NYS_ERR_UNSUPPORTED, "conv_kernel_size=%d: at most %d taps", conv_k, TAPS);
  }
  const int m_max = d == 128 ? 64 : 256;  // the token pass's LDS tiles bound M * d
  if (m != n && padded_m(m) > m_max)
    return fail(NYS_ERR_UNSUPPORTED, "backward: m=%d (up to %d landmarks at d=%d)", m, m_max, d);
  const size_t bytes = (size_t)B * H * n * d * sizeof(IO);
  const void* const ro[4] = {q, k, v, dout};
  void* const wr[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    if (reinterpret_cast<uintptr_t>(wr[i]) % 16 != 0) return fail(NYS_ERR_INVALID, "dq, dk, dv must be 16-byte aligned");
    for (int j = 0; j < 4; ++j)
      if (ranges_meet(wr[i], bytes, ro[j], bytes)) return fail(NYS_ERR_INVALID, "dq, dk, dv must not overlap q, k, v, dout");
    for (int j = 0; j < i; ++j)
      if (ranges_meet(wr[i], bytes, wr[j], bytes)) return fail(NYS_ERR_INVALID, "dq, dk, dv must not overlap");
  }
  for (const void* ptr : {q, k, v, dout})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return fail(NYS_ERR_INVALID, "q, k, v, dout must be 16-byte aligned");
  if (m == n) {
    switch (d) {
      case 32: return launch_backward_exact<IO, 32>(B, H, n, q, k, v, mask, conv_w, conv_k, dout, dq, dk, dv, dconv_w, st);
      case 64: return launch_backward_exact<IO, 64>(B, H, n, q, k, v, mask, conv_w, conv_k, dout, dq, dk, dv, dconv_w, st);
      default: return launch_backward_exact<IO, 128>(B, H, n, q, k, v, mask, conv_w, conv_k, dout, dq, dk, dv, dconv_w, st);
    }
  }
  Plan p = make_plan(B, H, n, m, d, (int)sizeof(IO));
  p.record = true;  // A is read back
  p.bwd = true;
  p.si = p.so = dense(B, H, n, d);
  const BwdPlan bp = make_bwd_plan(p, n_iter, conv_k, conv_w != nullptr);
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace* w = nullptr;
  rc = get_workspace(st, bp.total, &w);
  if (rc != NYS_OK) return rc;
#define NYS_BWD(MM, DD)                                                                                            \
  return launch_backward<IO, MM, DD>(p, bp, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, dout, dq, dk, dv, \
                                     dconv_w, st)
  switch (d * 1000 + p.m) {
    case 32032: NYS_BWD(32, 32);
    case 32064: NYS_BWD(64, 32);
    case 32096: NYS_BWD(96, 32);
    case 32128: NYS_BWD(128, 32);
    case 32160: NYS_BWD(160, 32);
    case 32192: NYS_BWD(192, 32);
    case 32224: NYS_BWD(224, 32);
    case 32256: NYS_BWD(256, 32);
    case 64032: NYS_BWD(32, 64);
    case 64064: NYS_BWD(64, 64);
    case 64096: NYS_BWD(96, 64);
    case 64128: NYS_BWD(128, 64);
    case 64160: NYS_BWD(160, 64);
    case 64192: NYS_BWD(192, 64);
    case 64224: NYS_BWD(224, 64);
    case 64256: NYS_BWD(256, 64);
    case 128032: NYS_BWD(32, 128);
    case 128064: NYS_BWD(64, 128);
    default: break;
  }
#undef NYS_BWD
  return fail(NYS_ERR_UNSUPPORTED, "backward: m=%d, d=%d", m, d);
}

}  // namespace host
}  // namespace nys
