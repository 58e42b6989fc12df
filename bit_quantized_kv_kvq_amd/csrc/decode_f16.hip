// decode_f16.hip -- decode kernel instantiations for f16 storage.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KERNEL_PTR(DT_F16)
}  // namespace dec
}  // namespace kvq
