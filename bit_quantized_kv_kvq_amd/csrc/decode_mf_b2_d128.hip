// decode_mf_b2_d128.hip -- matrix-core decode kernel instantiations for 2-bit codes and head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_MF_KERNEL_PTR(2, 128)
}  // namespace dec
}  // namespace kvq
