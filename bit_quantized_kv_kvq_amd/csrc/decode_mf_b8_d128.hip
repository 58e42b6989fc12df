// decode_mf_b8_d128.hip -- matrix-core decode kernel instantiations for 8-bit codes and head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_MF8_KERNEL_PTR(128)
}  // namespace dec
}  // namespace kvq
