// decode_mf_b2_d64.hip -- matrix-core decode kernel instantiations for 2-bit codes and head_dim 64.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_MF_KERNEL_PTR(2, 64)
}  // namespace dec
}  // namespace kvq
