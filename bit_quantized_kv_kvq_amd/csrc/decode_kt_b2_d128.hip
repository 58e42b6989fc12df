// decode_kt_b2_d128.hip -- decode kernel instantiations for per-token keys, 2-bit codes, head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(2, 128, KVQ_DECODE_KT_TABLE_D128(2))
}  // namespace dec
}  // namespace kvq
