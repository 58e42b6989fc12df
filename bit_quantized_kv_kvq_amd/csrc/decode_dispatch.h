// decode_dispatch.h -- instantiation table of the decode kernel for one storage
// dtype (included by decode_<dtype>.hip with KVQ_DT defined).
#pragma once
#include "decode_impl.h"

namespace kvq {
namespace dec {

template <int DT>
hipError_t launch_decode_dt(const DecArgs& a, int bits, int D, int gqa, int cpl, int tile, dim3 grid,
                            hipStream_t s);

template <>
hipError_t launch_decode_dt<DT_F32>(const DecArgs&, int, int, int, int, int, dim3, hipStream_t);
template <>
hipError_t launch_decode_dt<DT_BF16>(const DecArgs&, int, int, int, int, int, dim3, hipStream_t);
template <>
hipError_t launch_decode_dt<DT_F16>(const DecArgs&, int, int, int, int, int, dim3, hipStream_t);

// Channels per lane (CPL) by (head_dim, query heads per kv head, bits): wide lanes
// for MHA, narrower lanes when several query heads multiply the register state.
// The host picks the widest listed CPL that divides the value group size, so a
// lane's channels never straddle two value groups.
#define KVQ_DECODE_CASE(DT, BITS, D_, GQ_, CPL_, TILE_)                                           \
    if (bits == BITS && D == D_ && gqa == GQ_ && cpl == CPL_ && tile == TILE_) {                  \
        decode_kernel<DT, BITS, D_, GQ_, CPL_, TILE_><<<grid, kThreads, 0, s>>>(a);               \
        return hipGetLastError();                                                                 \
    }

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

#define KVQ_DEFINE_LAUNCH(DT)                                                                       \
    template <>                                                                                     \
    hipError_t launch_decode_dt<DT>(const DecArgs& a, int bits, int D, int gqa, int cpl, int tile,   \
                                    dim3 grid, hipStream_t s) {                                     \
        KVQ_DECODE_TABLE(DT)                                                                        \
        return hipErrorInvalidValue;                                                                \
    }

}  // namespace dec
}  // namespace kvq
