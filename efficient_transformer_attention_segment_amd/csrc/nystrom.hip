// Host side of libnystrom.so: argument validation, the per-(device, stream)
// workspace, the plan of each call and the C ABI declared in
// include/nystrom.h.  The launch sequences live in the kernel translation
// units (fwd_*.hip, exact.hip, bwd_*.hip; see host.hpp).
#include <cmath>
#include <functional>
#include <tuple>

#include "host.hpp"

// Device scratch of the allocation-free entry point (see static_scratch):
// one copy per device, for the life of the process.
static __device__ __align__(256) char scratch[NYS_NOALLOC_SCRATCH_BYTES];

namespace nys {
namespace host {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::mutex g_mu;
size_t g_ws_cap = 0;
unsigned g_spins = RENDEZVOUS_SPINS_DEFAULT;

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

Plan make_plan(int B, int H, int n, int mr, int d, int esize) {
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
  const int rg = bv_row_groups_for(esize, m, d);  // B V blocks per (head, chunk)
  const int target = std::max(p.BH, resident - p.npinv);
  int S = std::max(1, std::min(p.ntiles, target / (p.BH * rg)));
  p.tpc = (p.ntiles + S - 1) / S;
  p.S = (p.ntiles + p.tpc - 1) / p.tpc;
  const size_t BH = p.BH, M = m, D = d;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  p.off_zero = take(HEAD_BYTES);  // zero page, then the status word
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
    p.off_AT = take(BH * M * M * 4);
    p.off_Xt = take(BH * M * M * 4);
    p.off_X2t = take(BH * M * M * 4);
    p.off_Zt = take(BH * M * M * 4);
    p.off_Zt2 = take(BH * M * M * 4);
    p.off_colpart = take(BH * (M / 32) * M * 4);
    p.off_rowpart = take(BH * (M / 32) * 4);
  }
  p.total = o;
  return p;
}

std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::map<int, Side> g_side;

// Grow-only: a larger request waits for the stream (the old buffer may be in
// use by work already enqueued on it), then reallocates.
int get_workspace(hipStream_t st, size_t bytes, Workspace** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (g_ws_cap != 0 && bytes > g_ws_cap)
    return fail(NYS_ERR_HIP, "workspace of %zu bytes exceeds the cap of %zu bytes", bytes, g_ws_cap);
  Workspace& w = g_ws[{dev, st}];
  if (w.cap < bytes) {
    HIP_TRY(hipStreamSynchronize(st));
    if (w.buf) HIP_TRY(hipFree(w.buf));
    w.buf = nullptr;
    w.cap = 0;
    HIP_TRY(hipMalloc(&w.buf, bytes));
    w.cap = bytes;
    HIP_TRY(hipMemsetAsync(w.buf, 0, HEAD_BYTES, st));
  }
  *out = &w;
  return NYS_OK;
}

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
        void* probs = nullptr, Workspace* fixed = nullptr,
        const std::function<int(Plan&, Workspace*)>* pre = nullptr) {
  int rc = check_call(sizeof(IO), q, k, v, si, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, probs);
  if (rc != NYS_OK) return rc;
  if (fixed != nullptr && m != n) {
    const size_t need = make_plan(B, H, n, m, d, (int)sizeof(IO)).total;
    if (need > fixed->cap)
      return fail(NYS_ERR_UNSUPPORTED,
                  "this shape needs %zu bytes of scratch; the allocation-free entry point has %zu (NYS_NOALLOC_SCRATCH_BYTES)",
                  need, fixed->cap);
  }
  if (m == n) {
    if (d == 32) return launch_exact<IO, 32>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
    if (d == 128) return launch_exact<IO, 128>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
    return launch_exact<IO, 64>(B, H, n, si, so, q, k, v, mask, conv_w, conv_k, out, probs, st);
  }
  Plan p = make_plan(B, H, n, m, d, (int)sizeof(IO));
  p.record = pout != nullptr;  // the stage hook reads the intermediates back
  p.si = si;
  p.so = so;
  p.probs = probs;
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace* w = fixed;
  if (w == nullptr) {
    rc = get_workspace(st, p.total, &w);
    if (rc != NYS_OK) return rc;
  }
  if (pre != nullptr) {  // launches that write into the workspace first (the module's projection)
    rc = (*pre)(p, w);
    if (rc != NYS_OK) return rc;
  }
  rc = d == 32    ? dispatch_m<IO, 32>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st)
       : d == 128 ? dispatch_m<IO, 128>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st)
                  : dispatch_m<IO, 64>(p.m, p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st);
  if (wout) *wout = w;
  if (pout) *pout = p;
  return rc;
}

// --------------------------------------- allocation-free entry point ---
// nystrom_attention_noalloc runs the same launch sequence in a fixed scratch
// array instead of the grow-only workspace, for callers that cannot
// allocate.  Each device holds its own copy of the array (at its own
// address) from module load to process end; the host never passes the
// array's name to a kernel, only the address hipGetSymbolAddress gives for
// the current device.

// Fills n 16-byte words at p with zeros (a kernel rather than a memset, so
// a caller may capture it in a graph).
__global__ __launch_bounds__(256) void k_fill_zero(uint4* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_scratch_mu;
std::map<int, char*> g_scratch;  // device -> address of its scratch array

// The scratch array of the current device: its address is looked up once
// per device (with the device current), and at that first use the head of
// the array (the zero page every kernel reads as zero rows, and the status
// word) is cleared by a fill kernel on `st`.
int static_scratch(hipStream_t st, Workspace* out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(NYS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    if (reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
      return fail(NYS_ERR_HIP, "scratch array on device %d is not 256-byte aligned", dev);
    constexpr size_t words = HEAD_BYTES / 16;
    hipLaunchKernelGGL(k_fill_zero, dim3((words + 255) / 256), dim3(256), 0, st, static_cast<uint4*>(ptr), words);
    HIP_TRY(hipGetLastError());
    it = g_scratch.emplace(dev, static_cast<char*>(ptr)).first;
  }
  out->buf = it->second;
  out->cap = NYS_NOALLOC_SCRATCH_BYTES;
  return NYS_OK;
}

// ------------------------------------------- module: the q/k/v projection ---
// One hand-written GEMM (module.hip) writes x W^T + b as [B n, 3 H d] = [B, n,
// 3, H, d]; the attention kernels then read q, k, v from it in place through
// strides and write the context as [B, n, H d].

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
  if (b != nullptr && reinterpret_cast<uintptr_t>(b) % (4 * e) != 0)
    return fail(NYS_ERR_INVALID, "b_qkv must be aligned to 4 elements");
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
  // bf16, d = 64, landmarks a multiple of 32 and segments of L = n / m
  // tokens with L dividing 64: the projection forms the landmarks in its
  // epilogue (every 64-row output block holds whole segments of one
  // sequence) and the landmark pass is skipped
  const int L = n / m;
  const bool fold = sizeof(IO) == 2 && d == HD && m != n && m % 32 == 0 && L >= 2 && 64 % L == 0;
  if (m == n) {  // the exact branch takes no workspace
    rc = qkv_projection<IO>(x, w, b, (int)rows, hidden, (int)cols, qkv, st);
    if (rc != NYS_OK) return rc;
    return run<IO>(q, k, v, si, mask, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, st, nullptr,
                   nullptr);
  }
  // the projection runs once the workspace is known: the attention then
  // knows that q, k, v were just written (and where the landmarks are)
  const std::function<int(Plan&, Workspace*)> pre = [&](Plan& p, Workspace* ws) {
    const float s4 = 1.0f / sqrtf(sqrtf((float)HD));
    const QkvLandmarks lm{at<float>(ws, p.off_qt),  at<float>(ws, p.off_kt),  at<__bf16>(ws, p.off_qth),
                          at<__bf16>(ws, p.off_qtl), at<__bf16>(ws, p.off_kth), at<__bf16>(ws, p.off_ktl),
                          at<unsigned long long>(ws, p.off_slots), n, H, p.m, p.L, s4 / (float)p.L};
    const int r = qkv_projection<IO>(x, w, b, (int)rows, hidden, (int)cols, qkv, st, fold ? &lm : nullptr);
    if (r == NYS_OK) {
      p.landmarks_ready = fold;
      p.inputs_fresh = true;
    }
    return r;
  };
  return run<IO>(q, k, v, si, mask, conv_w, conv_k, so, B, H, n, d, m, n_iter, init_option, out, st, nullptr,
                 nullptr, nullptr, nullptr, &pre);
}

}  // namespace host
}  // namespace nys

using namespace nys;
using namespace nys::host;

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

__attribute__((visibility("default"))) int nystrom_attention_noalloc(
    int dtype, const void* q, const void* k, const void* v, long long in_batch_stride, long long in_head_stride,
    long long in_token_stride, const uint8_t* key_mask, const float* conv_w, int conv_kernel_size, int B, int H, int n,
    int d, int m, int n_iter, int init_option, void* out, long long out_batch_stride, long long out_head_stride,
    long long out_token_stride, struct ihipStream_t* stream) {
  try {
    g_err.clear();
    if (dtype != 0 && dtype != 1) return fail(NYS_ERR_INVALID, "dtype=%d is not 0 (float32) or 1 (bf16)", dtype);
    const Strides si{in_batch_stride, in_head_stride, in_token_stride};
    const Strides so{out_batch_stride, out_head_stride, out_token_stride};
    // every host-side check first: an invalid call touches nothing, not even the scratch
    int rc = check_call(dtype == 0 ? 4 : 2, q, k, v, si, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter,
                        init_option, out, nullptr);
    if (rc != NYS_OK) return rc;
    Workspace ws;
    rc = static_scratch(stream, &ws);
    if (rc != NYS_OK) return rc;
    if (dtype == 0)
      return run<float>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                        stream, nullptr, nullptr, nullptr, &ws);
    return run<u16>(q, k, v, si, key_mask, conv_w, conv_kernel_size, so, B, H, n, d, m, n_iter, init_option, out,
                    stream, nullptr, nullptr, nullptr, &ws);
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
    // with m > 128 the literal four-product iteration (float32 I/O, or more
    // than PINV_F16_MAX_ITER iterations) alternates between two buffers; the
    // expanded bf16 iteration updates Z in place
    const bool two_level = dtype == 1 && n_iter >= 1 && n_iter <= PINV_F16_MAX_ITER;
    size_t zoff = p.off_Z;
    if (M > 128 && !two_level && (n_iter % 2) == 1) zoff = p.off_Z2;
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

__attribute__((visibility("default"))) int nystrom_check_status(struct ihipStream_t* stream) {
  try {
    g_err.clear();
    HIP_TRY(hipStreamSynchronize(stream));
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    // the stream's workspace and the device's allocation-free scratch
    char* words[2] = {nullptr, nullptr};
    {
      std::lock_guard<std::mutex> lk(g_mu);
      auto it = g_ws.find({dev, stream});
      if (it != g_ws.end() && it->second.buf != nullptr) words[0] = it->second.buf + STATUS_OFF;
    }
    {
      std::lock_guard<std::mutex> lk(g_scratch_mu);
      auto it = g_scratch.find(dev);
      if (it != g_scratch.end()) words[1] = it->second + STATUS_OFF;
    }
    unsigned status = 0;
    for (char* word : words) {
      if (word == nullptr) continue;
      unsigned s = 0;
      HIP_TRY(hipMemcpy(&s, word, sizeof s, hipMemcpyDeviceToHost));
      if (s != 0) {
        const unsigned zero = 0;
        HIP_TRY(hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice));
      }
      status |= s;
    }
    if (status == 0) return NYS_OK;
    return fail(NYS_ERR_HIP,
                "a call on this stream gave up waiting for the pseudo-inverse blocks' rendezvous (original init): "
                "its scale c and output are NaN; the blocks were not all resident together");
  } catch (...) {
    return fail(NYS_ERR_HIP, "unexpected host exception");
  }
}

__attribute__((visibility("default"))) void nystrom_debug_set_rendezvous_spins(unsigned spins) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_spins = spins;
}

__attribute__((visibility("default"))) void nystrom_debug_set_workspace_cap(size_t bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_ws_cap = bytes;
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

