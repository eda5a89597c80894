// Forward Nystrom path, bf16 I/O, head size 64 (the tuned DMA and persistent output kernels).
#include "fwd_impl.hpp"

namespace nys {
namespace host {

template int dispatch_m<u16, 64>(int, const Plan&, Workspace*, const void*, const void*, const void*, const uint8_t*, const float*, int, int, int, void*, hipStream_t);

}  // namespace host
}  // namespace nys
