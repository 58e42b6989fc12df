// decode_sp_b4_d128.hip -- decode kernel instantiations for dense-and-sparse records,
// 4-bit codes and head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_SP_KERNEL_PTR(4, 128)
}  // namespace dec
}  // namespace kvq
