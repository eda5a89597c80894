// Forward Nystrom path, float32 I/O, head sizes 32 and 128.
#include "fwd_impl.hpp"

namespace nys {
namespace host {

template int dispatch_m<float, 32>(int, const Plan&, Workspace*, const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, void*, hipStream_t);
template int dispatch_m<float, 128>(int, const Plan&, Workspace*, const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, void*, hipStream_t);

}  // namespace host
}  // namespace nys
