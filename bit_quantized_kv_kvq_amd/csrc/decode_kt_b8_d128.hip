// decode_kt_b8_d128.hip -- decode kernel instantiations for per-token keys, 8-bit codes, head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(8, 128, KVQ_DECODE_KT8_TABLE_D128)
}  // namespace dec
}  // namespace kvq
