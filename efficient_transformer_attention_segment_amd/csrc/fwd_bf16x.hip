// Forward Nystrom path, bf16 I/O, head sizes 32 and 128.
#include "fwd_impl.hpp"

namespace nys {
namespace host {

template int dispatch_m<u16, 32>(int, const Plan&, Workspace*, const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, void*, hipStream_t);
template int dispatch_m<u16, 128>(int, const Plan&, Workspace*, const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, void*, hipStream_t);

}  // namespace host
}  // namespace nys
