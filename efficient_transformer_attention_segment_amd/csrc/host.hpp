// Host-side pieces shared by the translation units of libnystrom.so: error
// reporting, the per-call plan and workspace, the launch helper (optional
// per-kernel event timing) and the entry points each kernel translation unit
// provides.  The library is split so that the device code of the forward
// pass (per I/O type), the exact branch and the backward pass compile in
// parallel; every kernel template is instantiated in exactly one unit.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "nystrom.h"
#include "common.hpp"

namespace nys {
namespace host {

// ------------------------------------------------------------- errors ---
extern thread_local std::string g_err;
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

#define HIP_TRY(expr)                                                                                  \
  do {                                                                                                 \
    hipError_t e_ = (expr);                                                                            \
    if (e_ != hipSuccess) return ::nys::host::fail(NYS_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
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
  bool landmarks_ready = false;  // Qt, Kt (+ hi/lo) and the meeting slots already written (module fold)
  bool inputs_fresh = false;     // q, k, v written just before the call (the module's projection)
  size_t off_qt, off_kt, off_qth, off_qtl, off_kth, off_ktl, off_A, off_Z, off_colmax, off_rowmax, off_cscale;
  size_t off_pmax, off_psum, off_pacc, off_BV, off_W, off_wfh, off_wfl, off_X, off_T1, off_T2, off_Z2, off_zero;
  size_t off_slots, off_junk, off_lse;
  size_t off_AT, off_Xt, off_X2t, off_Zt, off_Zt2, off_colpart, off_rowpart;  // m > 128, bf16 I/O
  size_t total;
};

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t ZERO_BYTES = 4096;  // zero page at offset 0 of every workspace
// bf16 I/O: the pseudo-inverse iteration uses single fp16 products up to this
// many iterations and split-bf16 products beyond (the iterate's sensitivity
// to operand rounding grows with the iteration count).
constexpr int PINV_F16_MAX_ITER = 8;
// The pseudo-inverse blocks form their head's A themselves (no separate Gram
// launch) for the exact-coefficient init, and for the original init while
// they are few enough to be resident together for its one rendezvous.
constexpr int FUSED_GRAM_MAX_BLOCKS = 128;

// Landmark count of the kernels: the method's m rounded up to a multiple of
// 32.  The padding landmarks are zero rows of Qt and Kt, get no weight in
// any softmax over landmarks and zero rows in A, so they stay zero through
// the pseudo-inverse and contribute nothing to W or the output.
inline int padded_m(int m) { return (m + 31) & ~31; }

// esize: bytes per I/O element (the B V blocks' row groups depend on it; 4
// gives the largest workspace).
Plan make_plan(int B, int H, int n, int mr, int d, int esize = 4);

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
extern std::mutex g_prof_mu;
extern bool g_prof_on;
extern std::vector<ProfRec> g_prof;

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

// Guards the workspace map, the side streams and every launch sequence that
// uses a cached workspace.
extern std::mutex g_mu;
int get_workspace(hipStream_t st, size_t bytes, Workspace** out);
// Test hooks: a cap on the workspace size (0 = none; a larger request fails
// with NYS_ERR_HIP before anything is enqueued) and the rendezvous poll bound.
extern size_t g_ws_cap;
extern unsigned g_spins;
constexpr unsigned RENDEZVOUS_SPINS_DEFAULT = 1u << 20;  // about a second of polls
// Bytes at the start of every workspace that are cleared when it is
// allocated: the zero page, then the device status word (STATUS_OFF).
constexpr size_t STATUS_OFF = ZERO_BYTES;
constexpr size_t HEAD_BYTES = ZERO_BYTES + 256;

// A side stream per device, for work that can run beside the call's own
// stream (forked from it and joined back with events, so the caller sees one
// ordered sequence).  Default priority; non-blocking with respect to the
// null stream.  Guarded by g_mu.
struct Side {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, mid = nullptr, done = nullptr;
};
int get_side(Side** out);

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

// Dense [B, H, n, d] strides.
inline Strides dense(int B, int H, int n, int d) {
  (void)B;
  return Strides{(long long)H * n * d, (long long)n * d, d};
}

// Byte ranges [a, a + an) and [b, b + bn) intersect.
inline bool ranges_meet(const void* a, size_t an, const void* b, size_t bn) {
  const char* const pa = static_cast<const char*>(a);
  const char* const pb = static_cast<const char*>(b);
  return pa < pb + bn && pb < pa + an;
}

int validate(int esize, const void* q, const void* k, const void* v, int B, int H, int n, int d, int m, int n_iter,
             int init_option, const void* out);

// ------------------------------------------ kernel translation units ---
// Forward Nystrom launch sequence for the (padded) landmark count m, into the
// workspace w laid out by p (fwd_*.hip).
template <typename IO, int D>
int dispatch_m(int m, const Plan& p, Workspace* w, const void* q, const void* k, const void* v, const uint8_t* mask,
               const float* conv_w, int conv_k, int n_iter, int init_option, void* out, hipStream_t st);

// Exact branch (m == n), with the attention weights when probs != null
// (exact.hip).
template <typename IO, int D>
int launch_exact(int B, int H, int n, Strides si, Strides so, const void* q, const void* k, const void* v,
                 const uint8_t* mask, const float* conv_w, int conv_k, void* out, void* probs, hipStream_t st);

// The module's projection y = x W^T + b, [rows][cols] from x [rows][hidden]
// and W [cols][hidden] (module.hip); with lm != null (bf16 only) it also
// forms the landmarks in its epilogue.
template <typename IO>
int qkv_projection(const void* x, const void* w, const void* bias, int rows, int hidden, int cols, void* y,
                   hipStream_t st, const QkvLandmarks* lm = nullptr);

// The backward pass (bwd_*.hip).
template <typename IO>
int run_backward(const void* q, const void* k, const void* v, const uint8_t* mask, const float* conv_w, int conv_k,
                 int B, int H, int n, int d, int m, int n_iter, int init_option, const void* dout, void* dq, void* dk,
                 void* dv, float* dconv_w, hipStream_t st);

}  // namespace host
}  // namespace nys
