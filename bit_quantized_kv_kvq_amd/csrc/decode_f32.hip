// decode_f32.hip -- decode kernel instantiations for f32 storage.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KERNEL_PTR(DT_F32)
}  // namespace dec
}  // namespace kvq
