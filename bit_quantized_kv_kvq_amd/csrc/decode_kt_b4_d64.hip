// decode_kt_b4_d64.hip -- decode kernel instantiations for per-token keys, 4-bit codes, head_dim 64.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_KT_KERNEL_PTR(4, 64, KVQ_DECODE_KT_TABLE_D64(4))
}  // namespace dec
}  // namespace kvq
