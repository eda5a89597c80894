/*
 * nystrom.h -- C ABI of the MI355X (gfx950) Nystrom approximate
 * self-attention library (libnystrom.so).
 *
 * What it computes (pages cited by title and section):
 *   [P1] "Nystromformer 源码解析与实战指南：基于 Nystrom 采样的 O(n) 自注意力近似与
 *        Transformers 实现" (blog.gitcode.com);
 *   [P2] Hugging Face Transformers docs (zh), Nystromformer model page.
 *
 *   With Qs = q * d^-1/4 and Ks = k * d^-1/4            ([P1] 2.2),
 *   landmarks Qt, Kt = means of n/m contiguous tokens    ([P1] 2.3),
 *   F = softmax(Qs Kt^T), A = softmax(Qt Kt^T),
 *   B = softmax(Qt Ks^T + key mask)                      ([P1] 2.4),
 *   Z = n_iter steps of Z <- Z (13I - AZ(15I - AZ(7I - AZ))) / 4 from
 *       Z_0 = A^T / c                                     ([P1] 2.5),
 *   out = F (Z (B V)) + depthwise conv_w * V (65 taps, 'same')
 *                                                         ([P1] 2.4, 2.6).
 *   When m == n the exact attention softmax(Qs Ks^T + mask) V (+ conv) is
 *   computed instead ([P1] 2.1).
 *
 * Conventions shared by every entry point:
 *   - q, k, v, out are DEVICE pointers to [B, H, n, d] row-major tensors
 *     (d fastest).  The caller owns them.  out must not alias q, k or v.
 *   - key_mask is a DEVICE pointer to uint8 [B, n]: nonzero keeps a key,
 *     0 masks it ([P2] NystromformerModel.forward attention_mask).  NULL
 *     means no padding.  The mask enters B only (and the scores of the
 *     exact branch); padded tokens still enter the landmarks, F, A and the
 *     convolution.  A batch row with no kept key gets B V = 0, so its
 *     output is the convolution alone (no NaN).
 *   - conv_w is a DEVICE pointer to float32 [H, 65] (tap j multiplies V at
 *     token offset j - 32, zero outside [0, n); one filter per head shared
 *     by all d columns).  NULL disables the convolution ([P1] 2.6).
 *   - d (the head size) is 32, 64 or 128; 1 <= m <= 256 with n % m == 0,
 *     unless m == n (exact branch, any n >= 1).  Internally the
 *     landmarks are padded to a multiple of 32 with landmarks that take no
 *     weight anywhere, so any m in range gives the m-landmark result.
 *   - init_option 0 ("original", the default): c = (max column sum of A) *
 *     (max row sum of A), both maxima over every (batch, head) of the call.
 *     init_option 1 (exact coefficient): the same maxima per (batch, head).
 *     Ignored when m == n.
 *   - n_iter >= 0 (0 returns Z_0).  The pages' default is 6.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous: out is valid once the stream has synchronised.
 *     The library keeps one grow-only device workspace per (device, stream)
 *     behind a mutex; calls that share a stream are ordered by it.
 *   - Return value: NYS_OK, or a negative nys_status.  Every argument is
 *     validated on the host before anything is launched; on any error no
 *     kernel runs and out is not written.  nystrom_last_error() then holds
 *     a message (thread-local).
 */
#ifndef NYSTROM_H
#define NYSTROM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

typedef enum {
  NYS_OK = 0,
  NYS_ERR_INVALID = -1,     /* bad pointer, size or option */
  NYS_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle */
  NYS_ERR_HIP = -3          /* a HIP runtime call failed */
} nys_status;

enum { NYS_INIT_ORIGINAL = 0, NYS_INIT_EXACT = 1 };
enum { NYS_HEAD_DIM = 64, NYS_CONV_TAPS = 65, NYS_MAX_LANDMARKS = 256 };  /* NYS_HEAD_DIM: the pages' head size */

/* Nystrom attention, float32 q/k/v/out ([P1] 2.2-2.6; [P2] mask).
 * Errors: NYS_ERR_INVALID for NULL q/k/v/out, B/H/n/d/m <= 0, n % m != 0,
 * m > n, n_iter < 0, init_option not 0/1, out overlapping q/k/v;
 * NYS_ERR_UNSUPPORTED for d not 32, 64 or 128, m > 256 when m != n, or sizes whose
 * element counts overflow 2^31 per head;
 * NYS_ERR_HIP when a HIP call fails. */
int nystrom_attention(const float* q, const float* k, const float* v,
                      const uint8_t* key_mask, const float* conv_w,
                      int B, int H, int n, int d, int m, int n_iter,
                      int init_option, float* out,
                      struct ihipStream_t* stream);

/* Same operation and argument list with bfloat16 q/k/v/out (raw 16-bit
 * patterns, round-to-nearest-even on output); all accumulation is float32.
 * conv_w stays float32. */
int nystrom_attention_bf16(const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint8_t* key_mask,
                           const float* conv_w, int B, int H, int n, int d,
                           int m, int n_iter, int init_option, uint16_t* out,
                           struct ihipStream_t* stream);

/* The same two operations with the depthwise convolution's kernel size as
 * an argument (the pages' conv_kernel_size, [P1] 2.6 and 3.1; the calls
 * above fix it at 65).  conv_w is float32 [H, conv_kernel_size]: tap j
 * multiplies V at token offset j - conv_kernel_size / 2, zero outside
 * [0, n).  conv_kernel_size is read only when conv_w is not NULL.
 * Errors: those of nystrom_attention[_bf16], plus NYS_ERR_INVALID for an
 * even or non-positive conv_kernel_size ('same' padding needs a centre tap)
 * and NYS_ERR_UNSUPPORTED above 65 taps. */
int nystrom_attention_conv(const float* q, const float* k, const float* v,
                           const uint8_t* key_mask, const float* conv_w,
                           int conv_kernel_size, int B, int H, int n, int d,
                           int m, int n_iter, int init_option, float* out,
                           struct ihipStream_t* stream);
int nystrom_attention_bf16_conv(const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const uint8_t* key_mask,
                                const float* conv_w, int conv_kernel_size,
                                int B, int H, int n, int d, int m, int n_iter,
                                int init_option, uint16_t* out,
                                struct ihipStream_t* stream);

/* The general form: dtype 0 (float32 q/k/v/out) or 1 (bfloat16), the conv
 * kernel size as in nystrom_attention_conv, and q, k, v (one set of strides)
 * and out (another) as strided views of [B, H, n, d]: element
 * (b, h, t, c) of q is q[b * in_batch_stride + h * in_head_stride +
 * t * in_token_stride + c], in elements; the d channels of a token are
 * contiguous.  This reads, for example, q, k and v straight out of a fused
 * [B, n, 3, H, d] projection (strides n*3*H*d, d, 3*H*d) and writes out
 * as [B, n, H*d] (strides n*H*d, d, H*d), the module's layouts ([P1]
 * 2.7), with no transposes.  Errors: those of nystrom_attention_conv, plus
 * NYS_ERR_INVALID for a dtype other than 0/1, a pointer or stride that
 * breaks 16-byte alignment of the token rows, out strides under which two
 * (b, h, t) rows share an element, or out overlapping q, k or v. */
int nystrom_attention_ex(int dtype, const void* q, const void* k, const void* v,
                         long long in_batch_stride, long long in_head_stride,
                         long long in_token_stride, const uint8_t* key_mask,
                         const float* conv_w, int conv_kernel_size, int B, int H,
                         int n, int d, int m, int n_iter, int init_option, void* out,
                         long long out_batch_stride, long long out_head_stride,
                         long long out_token_stride, struct ihipStream_t* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * operation, arguments and errors of nystrom_attention_ex, with its
 * scratch in a fixed library-owned device array of
 * NYS_NOALLOC_SCRATCH_BYTES (one per device, held from the first call on
 * that device until the process ends) instead of the grow-only workspace.
 * The call allocates nothing (no hipMalloc, no hipFree, no allocating
 * library routine); the caller still owns q, k, v, key_mask, conv_w and
 * out.  Shapes whose scratch would exceed the array are rejected with
 * NYS_ERR_UNSUPPORTED before anything is enqueued (every workload up to
 * B H = 4 x 12 at n = 4096, m = 64, or n = 65536 at H = 4, m = 256, fits).
 * The first call on a device enqueues one small kernel on `stream` that
 * clears the head of the array.  Every call on a device shares that
 * device's array, and each call's kernels clear what they need zeroed;
 * calls that may overlap on one device (on different streams, or from
 * different threads) race on it, so the caller must order them. */
#define NYS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int nystrom_attention_noalloc(int dtype, const void* q, const void* k, const void* v,
                              long long in_batch_stride, long long in_head_stride,
                              long long in_token_stride, const uint8_t* key_mask,
                              const float* conv_w, int conv_kernel_size, int B, int H,
                              int n, int d, int m, int n_iter, int init_option, void* out,
                              long long out_batch_stride, long long out_head_stride,
                              long long out_token_stride, struct ihipStream_t* stream);

/* nystrom_attention_ex, and also the attention weights (output_attentions).
 *
 * Page [P1] section 2.4 names attention_probs = kernel_1 times the iterative
 * inverse of kernel_2, F Z, an n x m matrix whose rows are the approximate
 * attention weights; sections 2.7 and 5.3 say output_attentions returns
 * them (the full n x n softmax when the exact branch runs).  So:
 *   m <  n: probs [B, H, n, m] = F Z (the key mask does not enter F or A);
 *   m == n: probs [B, H, n, n] = softmax(q k^T / sqrt(d) + mask), masked
 *           keys 0, a row with no kept key all zeros.
 * probs is a dense DEVICE buffer of the call's dtype (float32 or bf16),
 * 16-byte aligned, owned by the caller, overlapping none of q, k, v and out.
 * Every other argument, and the output, as nystrom_attention_ex.  Errors:
 * as nystrom_attention_ex; NYS_ERR_INVALID also for a NULL, unaligned or
 * overlapping probs (nothing launched). */
int nystrom_attention_probs(int dtype, const void* q, const void* k, const void* v,
                            long long in_batch_stride, long long in_head_stride,
                            long long in_token_stride, const uint8_t* key_mask,
                            const float* conv_w, int conv_kernel_size, int B, int H,
                            int n, int d, int m, int n_iter, int init_option, void* out,
                            long long out_batch_stride, long long out_head_stride,
                            long long out_token_stride, void* probs,
                            struct ihipStream_t* stream);

/* The self-attention module around the core ([P1] section 2.2: q, k, v come
 * from three linear projections of the hidden states, split into heads as
 * (batch, heads, seq, head_dim); section 2.7: the context goes back to
 * (batch, seq, heads * head_dim)).
 *
 *   x      [B, n, hidden]      hidden states (16-byte aligned rows)
 *   w_qkv  [3 H d, hidden]     query, key and value weights stacked in that
 *                              order, each in nn.Linear's [out, in] layout
 *   b_qkv  [3 H d] or NULL     their biases
 *   qkv    [B, n, 3, H, d]     receives x w_qkv^T + b_qkv (one matrix-core
 *                              GEMM of this library, float32 accumulation,
 *                              rounded to the dtype);
 *                              the attention reads q, k, v from it in place
 *   out    [B, n, H d]         the context, head h in columns [h d, (h+1) d)
 * All in the dtype (0 float32, 1 bf16), dense, DEVICE memory owned by the
 * caller; qkv must not overlap x, w_qkv, b_qkv or out.  key_mask, conv_w,
 * conv_kernel_size, m, n_iter, init_option and the errors as
 * nystrom_attention_ex; every check runs before the GEMM is enqueued;
 * NYS_ERR_INVALID also for b_qkv not aligned to 4 elements. */
int nystrom_self_attention(int dtype, const void* x, const void* w_qkv, const void* b_qkv,
                           const uint8_t* key_mask, const float* conv_w, int conv_kernel_size,
                           int B, int n, int hidden, int H, int d, int m, int n_iter,
                           int init_option, void* qkv, void* out,
                           struct ihipStream_t* stream);

/* Backward pass for training ([P1] sections 2.2-2.6 differentiated; the
 * pages mention training with gradient checkpointing and the Trainer):
 * given dout = dL/dout for the output of the same call, writes
 * dq, dk, dv = dL/dq, dL/dk, dL/dv (the dtype's [B, H, n, d], dense) and,
 * when conv_w and dconv_w are both non-NULL, dconv_w = dL/dconv_w (float32
 * [H, conv_kernel_size]).  The intermediates are recomputed from q, k, v
 * (nothing is kept from the forward call).  The initial scale c is
 * differentiated through its maxima (the gradient of a maximum goes to its
 * first arg-max).  All pointers are DEVICE pointers owned by the caller;
 * dq, dk, dv must not overlap each other or q, k, v, dout.  Head sizes
 * d = 32, 64 and 128: the exact branch (m == n, any n) at each, the Nystrom
 * path with up to 256 landmarks at d = 32 and 64 and up to 64 at d = 128
 * (NYS_ERR_UNSUPPORTED for more).  Part of the work runs on a
 * library-owned side stream of the device (default priority), forked from
 * `stream` and joined back into it with events, so the call is ordered on
 * `stream` like any other; the first call on a device creates that stream
 * (nystrom_release destroys it).  Other errors as nystrom_attention. */
int nystrom_attention_backward(int dtype, const void* q, const void* k, const void* v,
                               const uint8_t* key_mask, const float* conv_w,
                               int conv_kernel_size, int B, int H, int n, int d, int m,
                               int n_iter, int init_option, const void* dout, void* dq,
                               void* dk, void* dv, float* dconv_w,
                               struct ihipStream_t* stream);

/* Bytes of device workspace a call of this shape uses (0 for invalid or
 * unsupported shapes). */
size_t nystrom_workspace_bytes(int B, int H, int n, int d, int m);

/* Message for the last non-OK return on this thread ("" if none). */
const char* nystrom_last_error(void);

/* Free every cached workspace (all devices and streams) and destroy the
 * backward pass's side streams.  Must not be called while work the library
 * enqueued may still be running. */
void nystrom_release(void);

/* Test hook: run the Nystrom path (m != n) like nystrom_attention[_bf16]
 * (dtype selects: 0 = float32 q/k/v/out, 1 = bfloat16) and, after the
 * stream has synchronised, copy the intermediate stages into the caller's
 * DEVICE buffers (float32, any may be NULL):
 *   qt, kt  [B,H,m,d]   landmarks of Qs, Ks          ([P1] 2.3)
 *   a       [B,H,m,m]   A = softmax(Qt Kt^T)          ([P1] 2.4)
 *   cscale  [B*H]       init scale c used for each head ([P1] 2.5)
 *   z       [B,H,m,m]   pseudo-inverse iterate after n_iter steps
 *   bv      [B,H,m,d]   B V                           ([P1] 2.4)
 *   w       [B,H,m,d]   Z (B V)
 * Synchronises `stream`.  Same errors as nystrom_attention; also
 * NYS_ERR_INVALID when m == n. */
int nystrom_debug_stages(int dtype, const void* q, const void* k,
                         const void* v, const uint8_t* key_mask,
                         const float* conv_w, int B, int H, int n, int d,
                         int m, int n_iter, int init_option, void* out,
                         float* qt, float* kt, float* a, float* cscale,
                         float* z, float* bv, float* w,
                         struct ihipStream_t* stream);

/* Device-side status of the work enqueued on `stream` ([P1] 2.5: the
 * original init's scale c is a maximum over every head, for which the
 * per-head pseudo-inverse blocks of one launch meet once; the wait is
 * bounded, and a block that gives up sets c to NaN, so its output is NaN,
 * and records the timeout in the stream's workspace).  Synchronises
 * `stream`, then returns NYS_OK, or NYS_ERR_HIP with a message in
 * nystrom_last_error() when a call on `stream` since the previous check
 * timed out (the record is cleared by the check).  The wait can only run
 * out when the blocks are not all resident together, e.g. when other work
 * fills the device's compute units. */
int nystrom_check_status(struct ihipStream_t* stream);

/* Test hooks for the failure paths (not for production use; both settings
 * are process-wide and stay until changed):
 *   nystrom_debug_set_rendezvous_spins: the bound on the rendezvous polls
 *     above (default 2^20, about a second; 0 makes every wait give up at
 *     once, so every kernel still exits normally);
 *   nystrom_debug_set_workspace_cap: a cap in bytes on the device workspace
 *     (0 = none); a call that needs more fails with NYS_ERR_HIP before
 *     anything is enqueued, so out is not written. */
void nystrom_debug_set_rendezvous_spins(unsigned spins);
void nystrom_debug_set_workspace_cap(size_t bytes);

/* Kernel timing for benchmarks (not part of the computation).  While
 * enabled (on != 0), every call brackets each kernel it launches with a
 * pair of hipEvents recorded on the call's stream.  nystrom_profile_collect
 * waits for those events, then writes up to `cap` entries: names[i] (static
 * strings: "k_landmark", "k_pinv_bv", "k_pinv_init", "k_pinv_gemm x4",
 * "k_merge", "k_out", "k_exact"), total_ms[i] (sum of elapsed times) and
 * launches[i], covering every launch since the previous collect; any of the
 * arrays may be NULL.  Returns the number of distinct kernels, or
 * NYS_ERR_HIP if an event could not be resolved. */
void nystrom_profile_enable(int on);
int nystrom_profile_collect(const char** names, double* total_ms, int* launches, int cap);

#ifdef __cplusplus
}
#endif

#endif /* NYSTROM_H */
