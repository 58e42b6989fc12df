// decode_mfsp_b2_d128.hip -- decode kernel instantiations for dense-and-sparse records on the
// matrix cores, 2-bit codes and head_dim 128.
#include "decode_dispatch.h"

namespace kvq {
namespace dec {
KVQ_DEFINE_MFSP_KERNEL_PTR(2)
}  // namespace dec
}  // namespace kvq
