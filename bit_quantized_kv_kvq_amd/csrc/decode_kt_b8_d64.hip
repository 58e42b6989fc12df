// decode_kt_b8_d64.hip -- decode kernel instantiations for per-token keys, 8-bit codes, head_dim 64.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(8, 64, KVQ_DECODE_KT8_TABLE_D64)
}  // namespace dec
}  // namespace kvq
