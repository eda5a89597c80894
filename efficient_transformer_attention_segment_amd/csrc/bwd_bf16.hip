// Backward pass, bf16 I/O.
#include "bwd_impl.hpp"

namespace nys {
namespace host {

template int run_backward<u16>(const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, int, int, int, int, int, const void*, void*, void*, void*, float*, hipStream_t);

}  // namespace host
}  // namespace nys
