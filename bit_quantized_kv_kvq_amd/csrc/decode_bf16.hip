// decode_bf16.hip -- decode kernel instantiations for bf16 storage.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KERNEL_PTR(DT_BF16)
}  // namespace dec
}  // namespace kvq
