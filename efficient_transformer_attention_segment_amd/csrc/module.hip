// The self-attention module's q/k/v projection (k_qkv.hpp) and its launch.
#include "host.hpp"
#include "k_qkv.hpp"

namespace nys {
namespace host {

template <typename IO>
int qkv_projection(const void* x, const void* w, const void* bias, int rows, int hidden, int cols, void* y,
                   hipStream_t st, const QkvLandmarks* lm) {
  QkvArgs a{x, w, bias, y, rows, cols, hidden, lm != nullptr ? 1 : 0, lm != nullptr ? *lm : QkvLandmarks{}};
  if (lm != nullptr && sizeof(IO) != 2) return fail(NYS_ERR_UNSUPPORTED, "landmarks in the projection need bf16 I/O");
  if constexpr (sizeof(IO) == 2) {
    HIP_TRY(allow_lds(k_qkv_bf16, QB_LDS));
    HIP_TRY(launch("k_qkv", k_qkv_bf16, dim3(qkv_grid(rows, cols, QB_BM, QB_BN)), dim3(QB_NT), (uint32_t)QB_LDS, st, a));
  } else {
    HIP_TRY(launch("k_qkv", k_qkv_f32, dim3(qkv_grid(rows, cols, QF_BM, QF_BN)), dim3(256), 0, st, a));
  }
  return NYS_OK;
}

template int qkv_projection<float>(const void*, const void*, const void*, int, int, int, void*, hipStream_t,
                                   const QkvLandmarks*);
template int qkv_projection<u16>(const void*, const void*, const void*, int, int, int, void*, hipStream_t,
                                 const QkvLandmarks*);

}  // namespace host
}  // namespace nys
