// decode_kt_b2_d64.hip -- decode kernel instantiations for per-token keys, 2-bit codes, head_dim 64.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(2, 64, KVQ_DECODE_KT_TABLE_D64(2))
}  // namespace dec
}  // namespace kvq
