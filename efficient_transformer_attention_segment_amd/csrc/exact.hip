// Exact branch (m == n): flash-style softmax attention with the key mask and
// the convolution, and on request the exact attention weights.
#include <cmath>

#include "host.hpp"
#include "k_bv.hpp"
#include "k_probs.hpp"

namespace nys {
namespace host {

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

template int launch_exact<float, 32>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                     const uint8_t*, const float*, int, void*, void*, hipStream_t);
template int launch_exact<float, 64>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                     const uint8_t*, const float*, int, void*, void*, hipStream_t);
template int launch_exact<float, 128>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                      const uint8_t*, const float*, int, void*, void*, hipStream_t);
template int launch_exact<u16, 32>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                   const uint8_t*, const float*, int, void*, void*, hipStream_t);
template int launch_exact<u16, 64>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                   const uint8_t*, const float*, int, void*, void*, hipStream_t);
template int launch_exact<u16, 128>(int, int, int, Strides, Strides, const void*, const void*, const void*,
                                    const uint8_t*, const float*, int, void*, void*, hipStream_t);

}  // namespace host
}  // namespace nys
