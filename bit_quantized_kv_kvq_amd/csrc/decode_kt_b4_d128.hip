// decode_kt_b4_d128.hip -- decode kernel instantiations for per-token keys, 4-bit codes, head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(4, 128, KVQ_DECODE_KT_TABLE_D128(4))
}  // namespace dec
}  // namespace kvq
