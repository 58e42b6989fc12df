// decode_dispatch.h -- instantiation table of the decode kernel for one storage
// dtype (included by decode_<dtype>.hip).
#pragma once
#include "decode_impl.h"

namespace kvq {
namespace dec {

// Kernel entry of the instantiation for (bits, head_dim, query heads per kv head,
// key channels per lane, tile), or nullptr if there is none.
template <int DT>
const void* decode_kernel_ptr(int bits, int D, int gqa, int cpl, int tile);

template <>
const void* decode_kernel_ptr<DT_F32>(int, int, int, int, int);
template <>
const void* decode_kernel_ptr<DT_BF16>(int, int, int, int, int);
template <>
const void* decode_kernel_ptr<DT_F16>(int, int, int, int, int);

// Key channels per lane (CPL): 32 for MHA with head_dim 128 (4 lanes per token),
// 16 when several query heads multiply the register state, 8 for 8 query heads
// with 4-bit codes.  The host picks CPL so that D / CPL lanes cover at least the
// value groups of a token (D / CPL >= D / G_V).
#define KVQ_DECODE_CASE(DT, BITS, D_, GQ_, CPL_, TILE_)                                     \
    if (bits == BITS && D == D_ && gqa == GQ_ && cpl == CPL_ && tile == TILE_)              \
        return reinterpret_cast<const void*>(&decode_kernel<DT, BITS, D_, GQ_, CPL_, TILE_>);

#define KVQ_DECODE_TILES(DT, BITS, D_, GQ_, CPL_) \
    KVQ_DECODE_CASE(DT, BITS, D_, GQ_, CPL_, 32)  \
    KVQ_DECODE_CASE(DT, BITS, D_, GQ_, CPL_, 64)

#define KVQ_DECODE_TABLE(DT)                 \
    KVQ_DECODE_TILES(DT, 4, 128, 1, 32)      \
    KVQ_DECODE_TILES(DT, 2, 128, 1, 32)      \
    KVQ_DECODE_TILES(DT, 4, 128, 1, 16)      \
    KVQ_DECODE_TILES(DT, 2, 128, 1, 16)      \
    KVQ_DECODE_TILES(DT, 4, 128, 2, 16)      \
    KVQ_DECODE_TILES(DT, 2, 128, 2, 16)      \
    KVQ_DECODE_TILES(DT, 4, 128, 4, 16)      \
    KVQ_DECODE_TILES(DT, 2, 128, 4, 16)      \
    KVQ_DECODE_TILES(DT, 4, 128, 8, 8)       \
    KVQ_DECODE_TILES(DT, 2, 128, 8, 16)      \
    KVQ_DECODE_TILES(DT, 4, 64, 1, 16)       \
    KVQ_DECODE_TILES(DT, 2, 64, 1, 16)       \
    KVQ_DECODE_TILES(DT, 4, 64, 2, 16)       \
    KVQ_DECODE_TILES(DT, 2, 64, 2, 16)       \
    KVQ_DECODE_TILES(DT, 4, 64, 4, 16)       \
    KVQ_DECODE_TILES(DT, 2, 64, 4, 16)       \
    KVQ_DECODE_TILES(DT, 4, 64, 8, 8)        \
    KVQ_DECODE_TILES(DT, 2, 64, 8, 16)

#define KVQ_DEFINE_KERNEL_PTR(DT)                                                        \
    template <>                                                                          \
    const void* decode_kernel_ptr<DT>(int bits, int D, int gqa, int cpl, int tile) {    \
        KVQ_DECODE_TABLE(DT)                                                             \
        return nullptr;                                                                  \
    }

}  // namespace dec
}  // namespace kvq
