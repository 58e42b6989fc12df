// decode_mf_b8_d64.hip -- matrix-core decode kernel instantiations for 8-bit codes and head_dim 64.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_MF8_KERNEL_PTR(64)
}  // namespace dec
}  // namespace kvq
