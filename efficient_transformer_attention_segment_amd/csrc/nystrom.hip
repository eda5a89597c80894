// Host side of libnystrom.so: argument validation, the per-(device, stream)
// workspace, the launch sequence and the C ABI declared in include/nystrom.h.
//
// Launch sequence for one Nystrom call (all on the caller's stream):
//   1 k_landmark   landmarks Qt, Kt (+ bf16 hi/lo)
//   2 k_gram       per head A = softmax(Qt Kt^T), its max column / row sum;
//                  only when the pseudo-inverse blocks cannot form A
//                  themselves (m > 128, or the original init with more
//                  heads than can meet in one resident round)
//   3 k_pinv_bv    one launch holding both the per-head pseudo-inverse
//                  blocks (m <= 128) and the B V partial blocks, so the
//                  pseudo-inverse chain runs beside the K/V stream
//     (m > 128: k_pinv_init + 4 k_pinv_gemm launches per iteration)
//   4 k_mw         B V from the partials, W = Z (B V) and its operand
//                  fragments
//   5 k_out_stream F W + conv(V) -> out (bf16 I/O; k_out for float32)
// Kernel boundaries are the only cross-workgroup synchronisation, apart
// from the one meeting of the pseudo-inverse blocks for the original init
// (data handed between workgroups of one launch across XCDs would need L2
// write-back and invalidation, which cost far more here than a launch).
// The exact branch (m == n) is one k_exact launch.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "nystrom.h"
#include "k_bv.hpp"
#include "k_landmark.hpp"
#include "k_merge.hpp"
#include "k_out.hpp"
#include "k_pinv.hpp"
#include "k_probs.hpp"
#include "k_bwd.hpp"

using namespace nys;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(NYS_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// ---------------------------------------------------------------- plan ---
struct Plan {
  int B, H, n, m, BH, L, RS, lpw, S, tpc, ntiles, npinv;
  int D;        // head size
  int mr;       // landmarks of the method; m is mr rounded up to a multiple of 32
  bool record;  // keep every intermediate in the workspace (stage hook)
  Strides si, so;  // element strides of q, k, v and of out
  void* probs;     // attention weights [B, H, n, mr] on request, else null
  bool bwd;        // forward stages for the backward pass: stop after W, keep B's normalisers
  size_t off_qt, off_kt, off_qth, off_qtl, off_kth, off_ktl, off_A, off_Z, off_colmax, off_rowmax, off_cscale;
  size_t off_pmax, off_psum, off_pacc, off_BV, off_W, off_wfh, off_wfl, off_X, off_T1, off_T2, off_Z2, off_zero;
  size_t off_slots, off_junk, off_lse;
  size_t total;
};

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t ZERO_BYTES = 4096;  // zero page at offset 0 of every workspace
// bf16 I/O: the pseudo-inverse iteration uses single fp16 products up to this
// many iterations and split-bf16 products beyond (the iterate's sensitivity
// to operand rounding grows with the iteration count).
constexpr int PINV_F16_MAX_ITER = 8;
// The pseudo-inverse blocks form their head's A themselves (no separate Gram
// launch) for the exact-coefficient init, and for the original init while
// they are few enough to be resident together for its one rendezvous.
constexpr int FUSED_GRAM_MAX_BLOCKS = 128;

int pow2floor(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}
int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Landmark count of the kernels: the method's m rounded up to a multiple of
// 32.  The padding landmarks are zero rows of Qt and Kt, get no weight in
// any softmax over landmarks and zero rows in A, so they stay zero through
// the pseudo-inverse and contribute nothing to W or the output.
int padded_m(int m) { return (m + 31) & ~31; }

Plan make_plan(int B, int H, int n, int mr, int d) {
  Plan p{};
  const int m = padded_m(mr);
  p.D = d;
  p.B = B;
  p.H = H;
  p.n = n;
  p.m = m;
  p.mr = mr;
  p.BH = B * H;
  p.L = n / mr;
  // landmark blocks: d / 8 threads per row, RS row slots per landmark, lpw
  // landmarks per block (at most 32, which divides m).  Eight rows per slot
  // where segments are long; for short segments enough slots (at most the
  // segment length) that the grid has about two blocks per CU.
  const int tpr = d / 8;
  const int rs_fill =
      std::min(pow2ceil((int)std::max(1LL, (2LL * 256 * 256) / ((long long)m * tpr * p.BH))), pow2floor(p.L));
  p.RS = std::min(256 / tpr, std::max({1, 256 / (tpr * 32), pow2floor(std::max(1, p.L / 8)), rs_fill}));
  p.lpw = 256 / (tpr * p.RS);
  // key chunks for the B V partials: as many blocks as stay resident in one
  // round next to the pseudo-inverse blocks (two blocks per CU)
  p.ntiles = (n + 31) / 32;  // the last tile is ragged when n % 32 != 0
  p.npinv = m <= 128 ? p.BH : 0;
  const int resident = 2 * 256;
  const int target = std::max(p.BH, resident - p.npinv);
  int S = std::max(1, std::min(p.ntiles, target / p.BH));
  p.tpc = (p.ntiles + S - 1) / S;
  p.S = (p.ntiles + p.tpc - 1) / p.tpc;
  const size_t BH = p.BH, M = m, D = d;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  p.off_zero = take(ZERO_BYTES);
  p.off_slots = take(BH * 16);
  p.off_junk = take(16 * HD * 2);  // output rows of tiles past a workgroup's range
  p.off_qt = take(BH * M * D * 4);
  p.off_kt = take(BH * M * D * 4);
  p.off_qth = take(BH * M * D * 2);
  p.off_qtl = take(BH * M * D * 2);
  p.off_kth = take(BH * M * D * 2);
  p.off_ktl = take(BH * M * D * 2);
  p.off_A = take(BH * M * M * 4);
  p.off_Z = take(BH * M * M * 4);
  p.off_colmax = take(BH * 4);
  p.off_rowmax = take(BH * 4);
  p.off_cscale = take(BH * 4);
  p.off_pmax = take(BH * p.S * M * 4);
  p.off_psum = take(BH * p.S * M * 4);
  p.off_pacc = take(BH * p.S * M * D * 4);
  p.off_BV = take(BH * M * D * 4);
  p.off_W = take(BH * M * D * 4);
  p.off_wfh = take(BH * M * D * 2);
  p.off_wfl = take(BH * M * D * 2);
  p.off_lse = take(BH * M * 4);
  if (m > 128) {
    p.off_X = take(BH * M * M * 4);
    p.off_T1 = take(BH * M * M * 4);
    p.off_T2 = take(BH * M * M * 4);
    p.off_Z2 = take(BH * M * M * 4);
  }
  p.total = o;
  return p;
}

// ------------------------------------------------------- kernel timing ---
// Every launch goes through launch().  While timing is enabled it uses
// hipExtLaunchKernelGGL with a start / stop event pair, which the runtime
// stamps with the kernel's own begin and end (no extra marker packets, so
// the figures match a kernel trace and the queue is not slowed);
// nystrom_profile_collect() resolves them into per-kernel sums.
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

template <typename... Args, typename F = void (*)(Args...)>
hipError_t launch(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                  Args... args) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on;
  }
  ProfRec rec{nullptr, nullptr, nullptr};
  if (on && hipEventCreate(&rec.a) == hipSuccess) {
    if (hipEventCreate(&rec.b) == hipSuccess)
      rec.name = name;
    else
      (void)hipEventDestroy(rec.a);
  }
  if (rec.name) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, rec.a, rec.b, 0, args...);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back(rec);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------- workspace ---
struct Workspace {
  char* buf = nullptr;
  size_t cap = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Grow-only: a larger request waits for the stream (the old buffer may be in
// use by work already enqueued on it), then reallocates.
int get_workspace(hipStream_t st, size_t bytes, Workspace** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  Workspace& w = g_ws[{dev, st}];
  if (w.cap < bytes) {
    HIP_TRY(hipStreamSynchronize(st));
    if (w.buf) HIP_TRY(hipFree(w.buf));
    w.buf = nullptr;
    w.cap = 0;
    HIP_TRY(hipMalloc(&w.buf, bytes));
    w.cap = bytes;
    HIP_TRY(hipMemsetAsync(w.buf, 0, ZERO_BYTES, st));
  }
  *out = &w;
  return NYS_OK;
}

// A side stream per device, for work that can run beside the call's own
// stream (forked from it and joined back with events, so the caller sees one
// ordered sequence).  Default priority; non-blocking with respect to the
// null stream.  Guarded by g_mu.
struct Side {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, mid = nullptr, done = nullptr;
};
std::map<int, Side> g_side;

int get_side(Side** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  Side& s = g_side[dev];
  if (s.st == nullptr) {
    HIP_TRY(hipStreamCreateWithFlags(&s.st, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&s.fork, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&s.join, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&s.mid, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&s.done, hipEventDisableTiming));
  }
  *out = &s;
  return NYS_OK;
}

template <typename T>
T* at(Workspace* w, size_t off) {
  return reinterpret_cast<T*>(w->buf + off);
}

template <typename F>
hipError_t allow_lds(F* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// --------------------------------------------------------- launches ---
template <typename IO, int M, int D>
int launch_nystrom(const Plan& p, Workspace* w, const void* q, const void* k, const void* v,
                   const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option, void* out,
                   hipStream_t st) {
  const float s4 = 1.0f / sqrtf(sqrtf((float)D));
  LandmarkArgs la;
  la.n = p.n;
  la.H = p.H;
  la.in = p.si;
  la.m = M;
  la.mr = p.mr;
  la.L = p.L;
  la.RS = p.RS;
  la.lpw = p.lpw;
  la.BH = p.BH;
  la.scale = s4 / (float)p.L;
  la.qt = at<float>(w, p.off_qt);
  la.kt = at<float>(w, p.off_kt);
  la.qt_hi = at<__bf16>(w, p.off_qth);
  la.qt_lo = at<__bf16>(w, p.off_qtl);
  la.kt_hi = at<__bf16>(w, p.off_kth);
  la.kt_lo = at<__bf16>(w, p.off_ktl);
  la.A = at<float>(w, p.off_A);
  la.colmax = at<float>(w, p.off_colmax);
  la.rowmax = at<float>(w, p.off_rowmax);
  la.slots = at<unsigned long long>(w, p.off_slots);
  HIP_TRY(launch("k_landmark", k_landmark<IO, M, D>, dim3(M / p.lpw, p.BH), dim3(256), 0, st, (const IO*)q,
                 (const IO*)k, la));
  // the pseudo-inverse blocks form A themselves only at d = 64 (their LDS
  // plan holds 64-channel landmarks)
  const bool fuse_gram = D == HD && M <= 128 && (init_option != 0 || p.npinv <= FUSED_GRAM_MAX_BLOCKS);
  if (!fuse_gram) {
    constexpr size_t glds = gram_lds_bytes<M, sizeof(IO) == 4, D>();
    HIP_TRY(allow_lds(k_gram<M, sizeof(IO) == 4, D>, glds));
    HIP_TRY(launch("k_gram", k_gram<M, sizeof(IO) == 4, D>, dim3(p.BH), dim3(64 * gram_waves<M>()), (uint32_t)glds,
                   st, la));
  }

  PinvArgs pa;
  pa.A = la.A;
  pa.colmax = la.colmax;
  pa.rowmax = la.rowmax;
  pa.Z = at<float>(w, p.off_Z);
  pa.cscale = at<float>(w, p.off_cscale);
  pa.BH = p.BH;
  pa.n_iter = n_iter;
  pa.init_option = init_option;
  pa.f16 = (sizeof(IO) == 2 && n_iter <= PINV_F16_MAX_ITER) ? 1 : 0;
  pa.fuse_gram = fuse_gram ? 1 : 0;
  pa.npinv = p.npinv;
  pa.record = p.record ? 1 : 0;
  pa.la = la;
  BvArgs ba;
  ba.k = k;
  ba.v = v;
  ba.key_mask = mask;
  ba.qt_hi = la.qt_hi;
  ba.qt_lo = la.qt_lo;
  ba.pmax = at<float>(w, p.off_pmax);
  ba.psum = at<float>(w, p.off_psum);
  ba.pacc = at<float>(w, p.off_pacc);
  ba.n = p.n;
  ba.H = p.H;
  ba.S = p.S;
  ba.tpc = p.tpc;
  ba.ntiles = p.ntiles;
  ba.lscale = s4;
  ba.in = p.si;
  size_t lds2 = (sizeof(IO) == 2 && D == HD) ? (size_t)DMA_LDS_BYTES : (size_t)KV<IO, D>::LDS_BYTES;
  lds2 = std::max<size_t>(lds2, bv_fold_bytes<M, D>());
  if constexpr (M <= 128)
    lds2 = std::max<size_t>(lds2, sizeof(IO) == 4 ? pinv_lds_bytes_f32<M>()
                                                  : std::max(pinv_lds_bytes<M, false>(), pinv_lds_bytes<M, true>()));
  // the padding-landmark and ragged-tile code only in the instance that needs it
  const bool pad = p.mr < M, edge = pad || p.n % 32 != 0;
  auto launch_bv = [&](auto kern) -> int {
    HIP_TRY(allow_lds(kern, lds2));
    HIP_TRY(launch("k_pinv_bv", kern, dim3(p.npinv + p.BH * p.S), dim3(64 * bv_waves<M>()), (uint32_t)lds2, st, pa,
                   ba, p.npinv));
    return NYS_OK;
  };
  const int brc = edge ? launch_bv(k_pinv_bv<IO, M, true, D>) : launch_bv(k_pinv_bv<IO, M, false, D>);
  if (brc != NYS_OK) return brc;

  const float* Zfinal = pa.Z;
  if constexpr (M > 128) {
    HIP_TRY(launch("k_pinv_init", k_pinv_init, dim3((M / 32) * (M / 32), p.BH), dim3(256), 0, st, pa, M));
    float* Zc = pa.Z;
    float* Zn = at<float>(w, p.off_Z2);
    float* X = at<float>(w, p.off_X);
    float* T1 = at<float>(w, p.off_T1);
    float* T2 = at<float>(w, p.off_T2);
    const dim3 gg((M / 32) * (M / 32), p.BH);
    for (int it = 0; it < n_iter; ++it) {
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)pa.A, (const float*)Zc, X,
                     0.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)X, (const float*)X, T1,
                     7.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)X, (const float*)T1, T2,
                     15.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)Zc, (const float*)T2, Zn,
                     13.f, 0.25f));
      std::swap(Zc, Zn);
    }
    Zfinal = Zc;
  }

  MergeArgs ma;
  ma.pmax = ba.pmax;
  ma.psum = ba.psum;
  ma.pacc = ba.pacc;
  ma.Z = Zfinal;
  ma.BV = at<float>(w, p.off_BV);
  ma.W = at<float>(w, p.off_W);
  ma.wf_hi = at<__bf16>(w, p.off_wfh);
  ma.wf_lo = at<__bf16>(w, p.off_wfl);
  ma.S = p.S;
  ma.BH = p.BH;
  ma.lse = p.bwd ? at<float>(w, p.off_lse) : nullptr;
  // threads per block: enough chunk subsets per row that each thread folds
  // one batch of 8 chunks (up to 1024 threads; 512 for m = 32)
  const int need = M * ((p.S + 7) / 8);
  // the bf16 output pass at d = 64 takes W^T in its own channel order
  constexpr bool B16 = sizeof(IO) == 2 && D == HD;
  constexpr int NT_MAX = M >= 64 ? 1024 : 512;
  const dim3 mwg(mw_blocks(p.BH, D));
  if (need <= 256)
    HIP_TRY(launch("k_mw", k_mw<M, B16, 256, D>, mwg, dim3(256), 0, st, ma));
  else if (need <= 512 || NT_MAX == 512)
    HIP_TRY(launch("k_mw", k_mw<M, B16, 512, D>, mwg, dim3(512), 0, st, ma));
  else
    HIP_TRY(launch("k_mw", k_mw<M, B16, NT_MAX, D>, mwg, dim3(NT_MAX), 0, st, ma));
  if (p.bwd) return NYS_OK;  // the backward pass takes it from here

  OutArgs oa;
  oa.q = q;
  oa.v = v;
  oa.zero = at<__bf16>(w, p.off_zero);
  oa.conv_w = conv_w;
  oa.conv_k = conv_k;
  oa.kt_hi = la.kt_hi;
  oa.kt_lo = la.kt_lo;
  oa.wf_hi = ma.wf_hi;
  oa.wf_lo = ma.wf_lo;
  oa.out = out;
  oa.n = p.n;
  oa.H = p.H;
  oa.lscale = s4;
  oa.in = p.si;
  oa.out_s = p.so;
  oa.mr = p.mr;
  if constexpr (sizeof(IO) == 2 && D == HD) {
    // persistent output pass: a token range of one head per workgroup, sized
    // so the grid fills the CUs at the occupancy its LDS allows in at most
    // one resident round (a second, partial round would cost a whole
    // workgroup lifetime)
    constexpr size_t lds4 = OutStreamLayout<M>::LDS_BYTES;
    constexpr int per_cu = std::min<int>(4, (int)(160 * 1024 / lds4));
    const int slots = 256 * per_cu;
    const int want = std::max(1, slots / p.BH);  // workgroups per head
    const int R = OUTS_UNIT * ((p.n + want * OUTS_UNIT - 1) / (want * OUTS_UNIT));
    const int nbh = (p.n + R - 1) / R;
    u16* const junk = at<u16>(w, p.off_junk);
    auto launch_out = [&](auto kern) -> int {
      HIP_TRY(launch("k_out_stream", kern, dim3(nbh, p.BH), dim3(256), 0u, st, oa, R, junk));
      return NYS_OK;
    };
    const int orc = conv_w != nullptr ? (pad ? launch_out(k_out_stream<M, true, true>)
                                             : launch_out(k_out_stream<M, true, false>))
                                      : (pad ? launch_out(k_out_stream<M, false, true>)
                                             : launch_out(k_out_stream<M, false, false>));
    if (orc != NYS_OK) return orc;
  } else {
    using OL = OutLayout<IO, M, D>;
    auto launch_out = [&](auto kern) -> int {
      HIP_TRY(allow_lds(kern, OL::LDS_BYTES));
      HIP_TRY(launch("k_out", kern, dim3((p.n + OL::TOK - 1) / OL::TOK, p.BH), dim3(256), (uint32_t)OL::LDS_BYTES, st,
                     oa));
      return NYS_OK;
    };
    const int orc = pad ? launch_out(k_out<IO, M, true, D>) : launch_out(k_out<IO, M, false, D>);
    if (orc != NYS_OK) return orc;
  }

  if (p.probs != nullptr) {
    ProbsArgs pr{};
    pr.q = q;
    pr.kt_hi = la.kt_hi;
    pr.kt_lo = la.kt_lo;
    pr.Z = Zfinal;
    pr.probs = p.probs;
    pr.n = p.n;
    pr.H = p.H;
    pr.mr = p.mr;
    pr.ldp = p.mr;
    pr.lscale = s4;
    pr.in = p.si;
    using PL = ProbsLayout<IO, M, D>;
    const int ntb = (p.n + PROBS_TOK - 1) / PROBS_TOK;
    const dim3 grid(((ntb + 7) / 8) * 8 * PL::NCB, p.BH);
    auto launch_probs = [&](auto kern) -> int {
      HIP_TRY(allow_lds(kern, PL::LDS_BYTES));
      HIP_TRY(launch("k_probs", kern, grid, dim3(256), (uint32_t)PL::LDS_BYTES, st, pr));
      return NYS_OK;
    };
    const int prc = pad ? launch_probs(k_probs<IO, M, true, D>) : launch_probs(k_probs<IO, M, false, D>);
    if (prc != NYS_OK) return prc;
  }
  return NYS_OK;
}

template <typename IO, int D>
int launch_exact(int B, int H, int n, Strides si, Strides so, const void* q, const void* k, const void* v,
                 const uint8_t* mask,
                 const float* conv_w, int conv_k, void* out, void* probs, hipStream_t st) {
  ExactArgs ea;
  ea.q = q;
  ea.k = k;
  ea.v = v;
  ea.key_mask = mask;
  ea.conv_w = conv_w;
  ea.conv_k = conv_k;
  ea.in = si;
  ea.out_s = so;
  ea.out = out;
  ea.n = n;
  ea.H = H;
  ea.lscale = 1.0f / sqrtf((float)D);
  const size_t lds = exact_lds_bytes<IO, D>();
  HIP_TRY(allow_lds(k_exact<IO, D>, lds));
  HIP_TRY(launch("k_exact", k_exact<IO, D>, dim3((n + 63) / 64, B * H), dim3(256), (uint32_t)lds, st, ea));
  if (probs != nullptr) {
    ProbsArgs pr{};
    pr.q = q;
    pr.k = k;
    pr.key_mask = mask;
    pr.probs = probs;
    pr.n = n;
    pr.H = H;
    pr.mr = n;
    pr.ldp = n;
    pr.lscale = ea.lscale;
    pr.in = si;
    constexpr int QB = 4 * xprobs_q<D>();
    HIP_TRY(launch("k_exact_probs", k_exact_probs<IO, D>, dim3((n + QB - 1) / QB, B * H), dim3(256), 0, st, pr));
  }
  return NYS_OK;
}

template <typename IO, int D>
int dispatch_m(int m, const Plan& p, Workspace* w, const void* q, const void* k, const void* v,
               const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option, void* out,
               hipStream_t st) {
#define NYS_M(MM) \
  case MM:        \
    return launch_nystrom<IO, MM, D>(p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st);
  switch (m) {
    NYS_M(32)
    NYS_M(64)
    NYS_M(96)
    NYS_M(128)
    NYS_M(160)
    NYS_M(192)
    NYS_M(224)
    NYS_M(256)
    default: break;
  }
#undef NYS_M
  return fail(NYS_ERR_UNSUPPORTED, "m=%d has no kernel instance", m);
}

// Dense [B, H, n, d] strides.
Strides dense(int B, int H, int n, int d) {
  (void)B;
  return Strides{(long long)H * n * d, (long long)n * d, d};
}

// A view's element range [lo, hi] (strides may be negative).
void view_range(const Strides& s, int B, int H, int n, int d, long long& lo, long long& hi) {
  lo = hi = 0;
  const long long ext[3][2] = {{s.b, B}, {s.h, H}, {s.t, n}};
  for (const auto& e : ext) (e[0] < 0 ? lo : hi) += e[0] * (e[1] - 1);
  hi += d - 1;
}

// Strides of q/k/v (si) and out (so): 16-byte aligned rows, and no two
// (batch, head, token) rows of out sharing an element (sorted by stride,
// each dimension must step over everything the smaller ones span).
int check_strides(int esize, const void* q, const void* k, const void* v, const void* out, Strides si, Strides so,
                  int B, int H, int n, int dh) {
  const int ext[3] = {B, H, n};
  for (const Strides* s : {&si, &so}) {
    const long long st[3] = {s->b, s->h, s->t};
    for (int i = 0; i < 3; ++i)
      if (ext[i] > 1 && (st[i] * esize) % 16 != 0)
        return fail(NYS_ERR_INVALID, "strides (%lld, %lld, %lld) elements: each must keep 16-byte row alignment",
                    s->b, s->h, s->t);
  }
  for (const void* ptr : {q, k, v, out})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return fail(NYS_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
  struct D {
    long long st;
    long long ex;
  } d[4] = {{1, dh}, {so.b < 0 ? -so.b : so.b, B}, {so.h < 0 ? -so.h : so.h, H}, {so.t < 0 ? -so.t : so.t, n}};
  std::sort(d, d + 4, [](const D& x, const D& y) { return x.st < y.st; });
  long long span = 0;
  for (const D& e : d) {
    if (e.ex <= 1) continue;
    if (e.st <= span) return fail(NYS_ERR_INVALID, "out strides (%lld, %lld, %lld) make rows overlap", so.b, so.h, so.t);
    span += e.st * (e.ex - 1);
  }
  long long olo, ohi, ilo, ihi;
  view_range(so, B, H, n, dh, olo, ohi);
  view_range(si, B, H, n, dh, ilo, ihi);
  const char* const ob = static_cast<const char*>(out);
  for (const void* ptr : {q, k, v}) {
    const char* const ib = static_cast<const char*>(ptr);
    if (ob + olo * esize <= ib + ihi * esize + (esize - 1) && ib + ilo * esize <= ob + ohi * esize + (esize - 1))
      return fail(NYS_ERR_INVALID, "out overlaps an input");
  }
  return NYS_OK;
}

// The weights buffer: dense [B, H, n, m] (n x n when m == n), 16-byte
// aligned, overlapping none of q, k, v and out.
int check_probs(int esize, const void* q, const void* k, const void* v, const void* out, const void* probs,
                Strides si, Strides so, int B, int H, int n, int d, int m) {
  if (reinterpret_cast<uintptr_t>(probs) % 16 != 0) return fail(NYS_ERR_INVALID, "probs must be 16-byte aligned");
  const char* const pb = static_cast<const char*>(probs);
  const char* const pe = pb + (size_t)B * H * n * m * esize;
  const void* const views[4] = {q, k, v, out};
  for (int i = 0; i < 4; ++i) {
    long long lo, hi;
    view_range(i < 3 ? si : so, B, H, n, d, lo, hi);
    const char* const b = static_cast<const char*>(views[i]);
    if (pb < b + (hi + 1) * esize && b + lo * esize < pe)
      return fail(NYS_ERR_INVALID, "probs overlaps %s", i < 3 ? "an input" : "out");
  }
  return NYS_OK;
}

int validate(int esize, const void* q, const void* k, const void* v, int B, int H, int n, int d, int m, int n_iter,
             int init_option, const void* out) {
  if (!q || !k || !v || !out) return fail(NYS_ERR_INVALID, "q, k, v and out must be non-NULL");
  if (B <= 0 || H <= 0 || n <= 0 || d <= 0 || m <= 0)
    return fail(NYS_ERR_INVALID, "B, H, n, d, m must be positive (got %d, %d, %d, %d, %d)", B, H, n, d, m);
  if (m > n) return fail(NYS_ERR_INVALID, "m=%d exceeds n=%d", m, n);
  if (n % m != 0) return fail(NYS_ERR_INVALID, "n=%d is not a multiple of m=%d", n, m);
  if (n_iter < 0) return fail(NYS_ERR_INVALID, "n_iter=%d is negative", n_iter);
  if (init_option != 0 && init_option != 1) return fail(NYS_ERR_INVALID, "init_option=%d is not 0 or 1", init_option);
  if (d != 32 && d != 64 && d != 128) return fail(NYS_ERR_UNSUPPORTED, "d=%d: head sizes 32, 64 and 128 are built", d);
  if ((long long)B * H > 65535) return fail(NYS_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)B * H);
  if ((long long)n * d >= (1LL << 31)) return fail(NYS_ERR_UNSUPPORTED, "n=%d too long", n);
  if (m != n) {
    if (m > NYS_MAX_LANDMARKS) return fail(NYS_ERR_UNSUPPORTED, "m=%d: at most 256 landmarks (unless m == n)", m);
  }
  (void)esize;
  return NYS_OK;
}

// Every host-side check of an attention call, before anything is enqueued.
int check_call(int esize, const void* q, const void* k, const void* v, Strides si, const float* conv_w, int conv_k,
               Strides so, int B, int H, int n, int d, int m, int n_iter, int init_option, const void* out,
               const void* probs) {
  int rc = validate(esize, q, k, v, B, H, n, d, m, n_iter, init_option, out);
  if (rc != NYS_OK) return rc;
  rc = check_strides(esize, q, k, v, out, si, so, B, H, n, d);
  if (rc != NYS_OK) return rc;
  if (probs != nullptr) {
    rc = check_probs(esize, q, k, v, out, probs, si, so, B, H, n, d, m);
    if (rc != NYS_OK) return rc;
  }
  if (conv_w != nullptr) {
    if (conv_k < 1 || conv_k % 2 == 0)
      return fail(NYS_ERR_INVALID, "conv_kernel_size=%d: 'same' padding needs an odd size >= 1", conv_k);
    if (conv_k > TAPS) return fail(NYS_ERR_UNSUPPORTED, "conv_kernel_size=%d: at most %d taps", conv_k, TAPS);
  }
  return NYS_OK;
}

template <typename IO>
int run(const void* q, const void* k, const void* v, Strides si, const uint8_t* mask, const float* conv_w, int conv_k,
        Strides so, int B,
        int H, int n,
        int d, int m, int n_iter, int init_option, void* out, hipStream_t st, Workspace** wout, Plan* pout,
        void* probs = nullptr) {
  int rc = check_call(sizeof(IO), q, k, v, si, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, probs);
  if (rc != NYS_OK) return rc;
  if (m == n) {
    if (d == 32) return launch_exact<IO, 32>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
    if (d == 128) return launch_exact<IO, 128>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
    return launch_exact<IO, 64>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
  }
  Plan p = make_plan(B, H, n, m, d);
  p.record = pout != nullptr;  // the stage hook reads the intermediates back
  p.si = si;
  p.so = so;
  p.probs = probs;
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace* w = nullptr;
  rc = get_workspace(st, p.total, &w);
  if (rc != NYS_OK) return rc;
  rc = d == 32    ? dispatch_m<IO, 32>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st)
       : d == 128 ? dispatch_m<IO, 128>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st)
                  : dispatch_m<IO, 64>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st);
  if (wout) *wout = w;
  if (pout) *pout = p;
  return rc;
}

// ------------------------------------------- module: the q/k/v projection ---
// One library GEMM (hipBLASLt) writes x W^T + b as [B n, 3 H d] = [B, n, 3,
// H, d]; the attention kernels then read q, k, v from it in place through
// strides and write the context as [B, n, H d].
struct LtPlan {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};
std::mutex g_lt_mu;
std::map<int, hipblasLtHandle_t> g_lt;                                         // per device
std::map<std::tuple<int, int, int, int, int, bool>, LtPlan> g_lt_plans;        // dev, dtype, rows, hidden, cols, bias
std::map<std::pair<int, hipStream_t>, Workspace> g_lt_ws;                      // GEMM workspace per stream
constexpr size_t LT_MAX_WS = 32u << 20;

#define LT_TRY(expr)                                                                                  \
  do {                                                                                              \
    hipblasStatus_t s_ = (expr);                                                                    \
    if (s_ != HIPBLAS_STATUS_SUCCESS) return fail(NYS_ERR_HIP, "%s: hipBLASLt status %d", #expr, (int)s_); \
  } while (0)

// y[rows][cols] = x[rows][hidden] W[cols][hidden]^T (+ bias[cols]), row-major,
// float32 accumulation.  In column-major terms y^T = op_T(W) x^T.
template <typename IO>
int qkv_projection(const void* x, const void* w, const void* bias, int rows, int hidden, int cols, void* y,
                   hipStream_t st) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_lt_mu);
  hipblasLtHandle_t& h = g_lt[dev];
  if (h == nullptr) LT_TRY(hipblasLtCreate(&h));
  const hipDataType t = sizeof(IO) == 4 ? HIP_R_32F : HIP_R_16BF;
  const auto key = std::make_tuple(dev, (int)sizeof(IO), rows, hidden, cols, bias != nullptr);
  auto it = g_lt_plans.find(key);
  if (it == g_lt_plans.end()) {
    LtPlan p;
    LT_TRY(hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F));
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta));
    LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb));
    if (bias != nullptr) {
      const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
      const int32_t bt = t;
      LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof epi));
      LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof bt));
      LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof bias));
    }
    LT_TRY(hipblasLtMatrixLayoutCreate(&p.la, t, hidden, cols, hidden));
    LT_TRY(hipblasLtMatrixLayoutCreate(&p.lb, t, hidden, rows, hidden));
    LT_TRY(hipblasLtMatrixLayoutCreate(&p.lc, t, cols, rows, cols));
    hipblasLtMatmulPreference_t pref = nullptr;
    LT_TRY(hipblasLtMatmulPreferenceCreate(&pref));
    const uint64_t wsmax = LT_MAX_WS;
    hipblasStatus_t s0 =
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax, sizeof wsmax);
    hipblasLtMatmulHeuristicResult_t res[1];
    int nres = 0;
    if (s0 == HIPBLAS_STATUS_SUCCESS)
      s0 = hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.lc, p.lc, pref, 1, res, &nres);
    (void)hipblasLtMatmulPreferenceDestroy(pref);
    LT_TRY(s0);
    if (nres < 1) return fail(NYS_ERR_UNSUPPORTED, "hipBLASLt has no algorithm for the %d x %d x %d projection", rows,
                              cols, hidden);
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    it = g_lt_plans.emplace(key, p).first;
  }
  LtPlan& p = it->second;
  if (bias != nullptr)
    LT_TRY(hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof bias));
  Workspace& ws = g_lt_ws[{dev, st}];
  if (ws.cap < p.ws) {
    HIP_TRY(hipStreamSynchronize(st));
    if (ws.buf) HIP_TRY(hipFree(ws.buf));
    ws.buf = nullptr;
    ws.cap = 0;
    HIP_TRY(hipMalloc(&ws.buf, p.ws));
    ws.cap = p.ws;
  }
  const float alpha = 1.f, beta = 0.f;
  LT_TRY(hipblasLtMatmul(h, p.op, &alpha, w, p.la, x, p.lb, &beta, y, p.lc, y, p.lc, &p.algo, ws.buf, p.ws, st));
  return NYS_OK;
}

// Byte ranges [a, a + an) and [b, b + bn) intersect.
bool ranges_meet(const void* a, size_t an, const void* b, size_t bn) {
  const char* const pa = static_cast<const char*>(a);
  const char* const pb = static_cast<const char*>(b);
  return pa < pb + bn && pb < pa + an;
}

template <typename IO>
int run_module(const void* x, const void* w, const void* b, const uint8_t* mask, const float* conv_w, int conv_k,
               int B, int n, int hidden, int H, int d, int m, int n_iter, int init_option, void* qkv, void* out,
               hipStream_t st) {
  if (!x || !w || !qkv || !out) return fail(NYS_ERR_INVALID, "x, w_qkv, qkv and out must be non-NULL");
  if (B <= 0 || n <= 0 || hidden <= 0 || H <= 0 || d <= 0)
    return fail(NYS_ERR_INVALID, "B, n, hidden, H, d must be positive (got %d, %d, %d, %d, %d)", B, n, hidden, H, d);
  const long long rows = (long long)B * n, cols = 3LL * H * d;
  if (rows > INT32_MAX || cols > INT32_MAX || rows * cols > (1LL << 40))
    return fail(NYS_ERR_UNSUPPORTED, "projection of %lld x %lld too large", rows, cols);
  const size_t e = sizeof(IO);
  if (((size_t)hidden * e) % 16 != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w) % 16 != 0 || reinterpret_cast<uintptr_t>(qkv) % 16 != 0)
    return fail(NYS_ERR_INVALID, "x, w_qkv and qkv must be 16-byte aligned with hidden * element size a multiple of 16");
  const size_t qkv_bytes = (size_t)rows * cols * e;
  if (ranges_meet(qkv, qkv_bytes, x, (size_t)rows * hidden * e) ||
      ranges_meet(qkv, qkv_bytes, w, (size_t)cols * hidden * e) ||
      (b != nullptr && ranges_meet(qkv, qkv_bytes, b, (size_t)cols * e)) ||
      ranges_meet(qkv, qkv_bytes, out, (size_t)rows * H * d * e))
    return fail(NYS_ERR_INVALID, "qkv overlaps x, w_qkv, b_qkv or out");
  const Strides si{n * cols, d, cols};
  const Strides so{(long long)n * H * d, d, (long long)H * d};
  const IO* const q = static_cast<const IO*>(qkv);
  const IO* const k = q + (size_t)H * d;
  const IO* const v = q + 2 * (size_t)H * d;
  int rc = check_call(e, q, k, v, si, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, nullptr);
  if (rc != NYS_OK) return rc;
  rc = qkv_projection<IO>(x, w, b, (int)rows, hidden, (int)cols, qkv, st);
  if (rc != NYS_OK) return rc;
  return run<IO>(q, k, v, si, mask, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, st, nullptr,
                 nullptr);
}

// ------------------------------------------------------------ backward ---
// Forward stages (without the output pass) into the plan's workspace, then
// the backward kernels into the regions that follow it.
struct BwdPlan {
  int nct, nck, ncv, mats;
  size_t off_dqf, off_pw, off_pk, off_pq, off_mm, off_dW, off_dBV, off_dQt, off_dKt, off_Dv, off_dc, off_cmax,
      off_cmaxj, off_rmax, off_dvc, off_pconv, total;
};

BwdPlan make_bwd_plan(const Plan& p, int n_iter, int conv_k, bool conv) {
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
  b.total = o;
  return b;
}

template <typename IO, int M, int D>
int launch_backward(const Plan& p, const BwdPlan& bp, Workspace* w, const void* q, const void* k, const void* v,
                    const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option,
                    const void* dout, void* dq, void* dk, void* dv, float* dconv_w, hipStream_t st) {
  int rc = launch_nystrom<IO, M, D>(p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, nullptr, st);
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
  // Side stream: for 64 landmarks the forward half of the per-head chain
  // (it needs only A) runs beside the token pass, which leaves CUs free;
  // then the conv's backward (it needs only dout, v and the weights) runs
  // beside the rest of the chain (one workgroup per head).  Both join back
  // before the kernels that read their results.
  constexpr bool SPLIT = M == 64;
  Side* sd = nullptr;
  if (SPLIT || conv_w != nullptr) {
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
  if constexpr (bwd_tok2(M, D)) {
    constexpr int tl = BwdTok2Layout<IO, M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_tok2<IO, M, D>, tl));
    HIP_TRY(launch("k_bwd_tok", k_bwd_tok2<IO, M, D>, dim3(bp.nct, p.BH), dim3(256), (uint32_t)tl, st, a));
  } else {
    constexpr int tl = BwdTokLayout<M, D>::BYTES;
    HIP_TRY(allow_lds(k_bwd_tok<IO, M, D>, tl));
    HIP_TRY(launch("k_bwd_tok", k_bwd_tok<IO, M, D>, dim3(bp.nct, p.BH), dim3(64 * bwd_tok_waves<M>()), (uint32_t)tl,
                   st, a));
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
  } else {
    HIP_TRY(allow_lds(k_bwd_mm1<M, D>, ml));
    HIP_TRY(launch("k_bwd_mm1", k_bwd_mm1<M, D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)ml, st, a));
  }
  HIP_TRY(allow_lds(k_bwd_mm2<M, D>, ml));
  HIP_TRY(launch("k_bwd_mm2", k_bwd_mm2<M, D>, dim3(p.BH), dim3(BWD_MM_NT), (uint32_t)ml, st, a));
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
  if (conv_w != nullptr && dconv_w != nullptr)
    HIP_TRY(launch("k_bwd_wsum", k_bwd_wsum, dim3(p.H), dim3(1024), 0, st, a));
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
  take(ZERO_BYTES);
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
  const int m_max = d == 128 ? 64 : 128;  // the token pass's LDS tiles bound M * d
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
  Plan p = make_plan(B, H, n, m, d);
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
    case 64032: NYS_BWD(32, 64);
    case 64064: NYS_BWD(64, 64);
    case 64096: NYS_BWD(96, 64);
    case 64128: NYS_BWD(128, 64);
    case 128032: NYS_BWD(32, 128);
    case 128064: NYS_BWD(64, 128);
    default: break;
  }
#undef NYS_BWD
  return fail(NYS_ERR_UNSUPPORTED, "backward: m=%d, d=%d", m, d);
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int nystrom_attention(const float* q, const float* k, const float* v,
                                                             const uint8_t* key_mask, const float* conv_w, int B,
                                                             int H, int n, int d, int m, int n_iter,
                                                             int init_option, float* out,
                                                             struct ihipStream_t* stream) {
  try {
    g_err.clear();
    return run<float>(q, k, v, dense(B, H, n, d), key_mask, conv_w, TAPS, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream, nullptr,
                      nullptr);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_bf16(const uint16_t* q, const uint16_t* k,
                                                                  const uint16_t* v, const uint8_t* key_mask,
                                                                  const float* conv_w, int B, int H, int n, int d,
                                                                  int m, int n_iter, int init_option, uint16_t* out,
                                                                  struct ihipStream_t* stream) {
  try {
    g_err.clear();
    return run<u16>(q, k, v, dense(B, H, n, d), key_mask, conv_w, TAPS, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream, nullptr,
                    nullptr);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_conv(const float* q, const float* k, const float* v,
                                                                  const uint8_t* key_mask, const float* conv_w,
                                                                  int conv_kernel_size, int B, int H, int n, int d,
                                                                  int m, int n_iter, int init_option, float* out,
                                                                  struct ihipStream_t* stream) {
  try {
    g_err.clear();
    return run<float>(q, k, v, dense(B, H, n, d), key_mask, conv_w, conv_kernel_size, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream,
                      nullptr, nullptr);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_bf16_conv(const uint16_t* q, const uint16_t* k,
                                                                       const uint16_t* v, const uint8_t* key_mask,
                                                                       const float* conv_w, int conv_kernel_size,
                                                                       int B, int H, int n, int d, int m, int n_iter,
                                                                       int init_option, uint16_t* out,
                                                                       struct ihipStream_t* stream) {
  try {
    g_err.clear();
    return run<u16>(q, k, v, dense(B, H, n, d), key_mask, conv_w, conv_kernel_size, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream,
                    nullptr, nullptr);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_ex(
    int dtype, const void* q, const void* k, const void* v, long long in_batch_stride, long long in_head_stride,
    long long in_token_stride, const uint8_t* key_mask, const float* conv_w, int conv_kernel_size, int B, int H, int n,
    int d, int m, int n_iter, int init_option, void* out, long long out_batch_stride, long long out_head_stride,
    long long out_token_stride, struct ihipStream_t* stream) {
  try {
    g_err.clear();
    const Strides si{in_batch_stride, in_head_stride, in_token_stride};
    const Strides so{out_batch_stride, out_head_stride, out_token_stride};
    if (dtype == 0)
      return run<float>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                        stream, nullptr, nullptr);
    if (dtype == 1)
      return run<u16>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                      stream, nullptr, nullptr);
    return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_probs(
    int dtype, const void* q, const void* k, const void* v, long long in_batch_stride, long long in_head_stride,
    long long in_token_stride, const uint8_t* key_mask, const float* conv_w, int conv_kernel_size, int B, int H, int n,
    int d, int m, int n_iter, int init_option, void* out, long long out_batch_stride, long long out_head_stride,
    long long out_token_stride, void* probs, struct ihipStream_t* stream) {
  try {
    g_err.clear();
    if (probs == nullptr) return fail(NYS_ERR_INVALID, "probs must be non-NULL");
    const Strides si{in_batch_stride, in_head_stride, in_token_stride};
    const Strides so{out_batch_stride, out_head_stride, out_token_stride};
    if (dtype == 0)
      return run<float>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                        stream, nullptr, nullptr, probs);
    if (dtype == 1)
      return run<u16>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                      stream, nullptr, nullptr, probs);
    return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_self_attention(
    int dtype, const void* x, const void* w_qkv, const void* b_qkv, const uint8_t* key_mask, const float* conv_w,
    int conv_kernel_size, int B, int n, int hidden, int H, int d, int m, int n_iter, int init_option, void* qkv,
    void* out, struct ihipStream_t* stream) {
  try {
    g_err.clear();
    if (dtype == 0)
      return run_module<float>(x, w_qkv, b_qkv, key_mask, conv_w, conv_kernel_size, B, n, hidden, H, d, m, n_iter,
                               init_option, qkv, out, stream);
    if (dtype == 1)
      return run_module<u16>(x, w_qkv, b_qkv, key_mask, conv_w, conv_kernel_size, B, n, hidden, H, d, m, n_iter,
                             init_option, qkv, out, stream);
    return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) int nystrom_attention_backward(
    int dtype, const void* q, const void* k, const void* v, const uint8_t* key_mask, const float* conv_w,
    int conv_kernel_size, int B, int H, int n, int d, int m, int n_iter, int init_option, const void* dout, void* dq,
    void* dk, void* dv, float* dconv_w, struct ihipStream_t* stream) {
  try {
    g_err.clear();
    if (dtype == 0)
      return run_backward<float>(q, k, v, key_mask, conv_w, conv_kernel_size, B, H, n, d, m, n_iter, init_option,
                                 dout, dq, dk, dv, dconv_w, stream);
    if (dtype == 1)
      return run_backward<u16>(q, k, v, key_mask, conv_w, conv_kernel_size, B, H, n, d, m, n_iter, init_option, dout,
                               dq, dk, dv, dconv_w, stream);
    return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) size_t nystrom_workspace_bytes(int B, int H, int n, int d, int m) {
  if (B <= 0 || H <= 0 || n <= 0 || (d != 32 && d != 64 && d != 128) || m <= 0 || m > n || n % m != 0) return 0;
  if (m == n) return 0;
  if (m > NYS_MAX_LANDMARKS) return 0;
  return make_plan(B, H, n, m, d).total;
}

__attribute__((visibility("default"))) const char* nystrom_last_error(void) { return g_err.c_str(); }

__attribute__((visibility("default"))) void nystrom_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& kv : g_ws) {
    if (kv.second.buf) (void)hipFree(kv.second.buf);
  }
  g_ws.clear();
  for (auto& kv : g_side) {
    (void)hipStreamDestroy(kv.second.st);
    (void)hipEventDestroy(kv.second.fork);
    (void)hipEventDestroy(kv.second.join);
    (void)hipEventDestroy(kv.second.mid);
    (void)hipEventDestroy(kv.second.done);
  }
  g_side.clear();
  std::lock_guard<std::mutex> lk2(g_lt_mu);
  for (auto& kv : g_lt_ws) {
    if (kv.second.buf) (void)hipFree(kv.second.buf);
  }
  g_lt_ws.clear();
}

__attribute__((visibility("default"))) int nystrom_debug_stages(int dtype, const void* q, const void* k,
                                                                const void* v, const uint8_t* key_mask,
                                                                const float* conv_w, int B, int H, int n, int d,
                                                                int m, int n_iter, int init_option, void* out,
                                                                float* qt, float* kt, float* a, float* cscale,
                                                                float* z, float* bv, float* wout,
                                                                struct ihipStream_t* stream) {
  try {
    g_err.clear();
    if (dtype != 0 && dtype != 1) return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
    if (m == n) return fail(NYS_ERR_INVALID, "stages exist only on the Nystrom path (m != n)");
    Workspace* w = nullptr;
    Plan p{};
    int rc = dtype == 0
                 ? run<float>(q, k, v, dense(B, H, n, d), key_mask, conv_w, TAPS, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream, &w, &p)
                 : run<u16>(q, k, v, dense(B, H, n, d), key_mask, conv_w, TAPS, dense(B, H, n, d), B, H, n, d, m, n_iter, init_option, out, stream, &w, &p);
    if (rc != NYS_OK) return rc;
    HIP_TRY(hipStreamSynchronize(stream));
    std::lock_guard<std::mutex> lk(g_mu);
    const size_t BH = p.BH, M = p.m, mr = p.mr;  // workspace rows M, caller rows mr
    // after n_iter > 0 with m > 128 the final iterate lives in one of two buffers
    size_t zoff = p.off_Z;
    if (M > 128 && (n_iter % 2) == 1) zoff = p.off_Z2;
    char* const base = static_cast<char*>(w->buf);
    // [BH][M][d] -> [BH][mr][d]
    struct Rows {
      float* dst;
      size_t off;
    } rows[] = {{qt, p.off_qt}, {kt, p.off_kt}, {bv, p.off_BV}, {wout, p.off_W}};
    for (const Rows& r : rows)
      if (r.dst)
        HIP_TRY(hipMemcpy2DAsync(r.dst, mr * p.D * 4, base + r.off, M * p.D * 4, mr * p.D * 4, BH,
                                 hipMemcpyDeviceToDevice, stream));
    // [BH][M][M] -> [BH][mr][mr]
    struct Mats {
      float* dst;
      size_t off;
    } mats[] = {{a, p.off_A}, {z, zoff}};
    for (const Mats& mt : mats)
      if (mt.dst)
        for (size_t h = 0; h < BH; ++h)
          HIP_TRY(hipMemcpy2DAsync(mt.dst + h * mr * mr, mr * 4, base + mt.off + h * M * M * 4, M * 4, mr * 4, mr,
                                   hipMemcpyDeviceToDevice, stream));
    if (cscale) HIP_TRY(hipMemcpyAsync(cscale, base + p.off_cscale, BH * 4, hipMemcpyDeviceToDevice, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    return NYS_OK;
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) void nystrom_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
}

__attribute__((visibility("default"))) int nystrom_profile_collect(const char** names, double* total_ms,
                                                                   int* launches, int cap) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof);
  }
  std::vector<const char*> nm;
  std::vector<double> tot;
  std::vector<int> cnt;
  int rc = 0;
  for (const ProfRec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = NYS_ERR_HIP;
    size_t i = 0;
    while (i < nm.size() && std::strcmp(nm[i], r.name) != 0) ++i;
    if (i == nm.size()) {
      nm.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  if (rc != 0) return fail(rc, "hipEvent timing failed");
  const int k = (int)std::min<size_t>(nm.size(), cap < 0 ? 0 : (size_t)cap);
  for (int i = 0; i < k; ++i) {
    if (names) names[i] = nm[i];
    if (total_ms) total_ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return (int)nm.size();
}

}  // extern "C"
