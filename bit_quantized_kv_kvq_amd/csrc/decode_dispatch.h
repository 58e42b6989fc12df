// decode_dispatch.h -- instantiation table of the decode kernel (included by
// decode_b<bits>_d<head_dim>.hip).
#pragma once
#include "decode_impl.h"

namespace kvq {
namespace dec {

// Kernel entry of the instantiation for (query heads per kv head, key channels
// per lane, tile, tiles per key group) at a code width and head_dim, or nullptr
// if there is none.  Defined in decode_b<bits>_d<head_dim>.hip.
template <int BITS, int D>
const void* decode_kernel_ptr(int gqa, int cpl, int tile, int tpg);

// Matrix-core stream (several query heads per kv head): kernel entry for (query
// heads per kv head, 64-token tiles per key group, value groups per token), or
// nullptr.  Defined in decode_mf_b<bits>_d<head_dim>.hip.
template <int BITS, int D>
const void* decode_mf_kernel_ptr(int gqa, int tpg, int nvg);

// Dense-and-sparse records (one outlier per quantization vector), on the VALU
// stream: kernel entry for (query heads per kv head, key channels per lane, tile,
// tiles per key group, value groups per token), or nullptr.  Defined in
// decode_sp_b<bits>_d<head_dim>.hip.
template <int BITS, int D>
const void* decode_sp_kernel_ptr(int gqa, int cpl, int tile, int tpg, int nvg);

// Dense-and-sparse records on the matrix cores (several query heads per kv head,
// head_dim 128): entry for (query heads per kv head, 64-token tiles per key group,
// value groups per token), or nullptr.  Defined in decode_mfsp_b<bits>_d128.hip.
template <int BITS>
const void* decode_mfsp_kernel_ptr(int gqa, int tpg, int nvg);
// Per-token keys: the VALU stream (one query head per kv head, 2- and 4-bit codes,
// 64-token tiles) when mf is false, the matrix-core stream otherwise; entry for
// (query heads per kv head, key channels per lane, 64-token tiles per key group,
// value groups per token), or nullptr.  Defined in decode_kt_b<bits>_d<head_dim>.hip.
template <int BITS, int D>
const void* decode_kt_kernel_ptr(int gqa, int cpl, int tpg, int nvg, bool mf);
template <>
const void* decode_kt_kernel_ptr<2, 128>(int, int, int, int, bool);
template <>
const void* decode_kt_kernel_ptr<4, 128>(int, int, int, int, bool);
template <>
const void* decode_kt_kernel_ptr<8, 128>(int, int, int, int, bool);
template <>
const void* decode_kt_kernel_ptr<2, 64>(int, int, int, int, bool);
template <>
const void* decode_kt_kernel_ptr<4, 64>(int, int, int, int, bool);
template <>
const void* decode_kt_kernel_ptr<8, 64>(int, int, int, int, bool);

template <>
const void* decode_mfsp_kernel_ptr<4>(int, int, int);
template <>
const void* decode_mfsp_kernel_ptr<2>(int, int, int);

template <>
const void* decode_sp_kernel_ptr<4, 128>(int, int, int, int, int);
template <>
const void* decode_sp_kernel_ptr<2, 128>(int, int, int, int, int);
template <>
const void* decode_sp_kernel_ptr<4, 64>(int, int, int, int, int);
template <>
const void* decode_sp_kernel_ptr<2, 64>(int, int, int, int, int);

template <>
const void* decode_kernel_ptr<4, 128>(int, int, int, int);
template <>
const void* decode_kernel_ptr<2, 128>(int, int, int, int);
template <>
const void* decode_kernel_ptr<4, 64>(int, int, int, int);
template <>
const void* decode_kernel_ptr<2, 64>(int, int, int, int);
template <>
const void* decode_mf_kernel_ptr<4, 128>(int, int, int);
template <>
const void* decode_mf_kernel_ptr<2, 128>(int, int, int);
template <>
const void* decode_mf_kernel_ptr<4, 64>(int, int, int);
template <>
const void* decode_mf_kernel_ptr<2, 64>(int, int, int);
template <>
const void* decode_mf_kernel_ptr<8, 128>(int, int, int);
template <>
const void* decode_mf_kernel_ptr<8, 64>(int, int, int);

// Key channels per lane (CPL): 32 for MHA with head_dim 128 (4 lanes per token),
// 16 when several query heads multiply the register state, 8 for 8 query heads
// with 4-bit codes.  The host picks CPL so that D / CPL lanes cover at least the
// value groups of a token (D / CPL >= D / G_V).  Tiles are 64 tokens for one
// query head per kv head and 32 otherwise; key groups of 32 to 256 tokens.
#define KVQ_DECODE_CASE(BITS, D_, GQ_, CPL_, TILE_, TPG_)                     \
    if (gqa == GQ_ && cpl == CPL_ && tile == TILE_ && tpg == TPG_)           \
        return reinterpret_cast<const void*>(&decode_kernel<BITS, D_, GQ_, CPL_, TILE_, TPG_>);

#define KVQ_DECODE_GROUPS_MHA(BITS, D_, CPL_)     \
    KVQ_DECODE_CASE(BITS, D_, 1, CPL_, 32, 1)     \
    KVQ_DECODE_CASE(BITS, D_, 1, CPL_, 64, 1)     \
    KVQ_DECODE_CASE(BITS, D_, 1, CPL_, 64, 2)     \
    KVQ_DECODE_CASE(BITS, D_, 1, CPL_, 64, 4)

#define KVQ_DECODE_GROUPS_GQA(BITS, D_, GQ_, CPL_) \
    KVQ_DECODE_CASE(BITS, D_, GQ_, CPL_, 32, 1)    \
    KVQ_DECODE_CASE(BITS, D_, GQ_, CPL_, 32, 2)    \
    KVQ_DECODE_CASE(BITS, D_, GQ_, CPL_, 32, 4)    \
    KVQ_DECODE_CASE(BITS, D_, GQ_, CPL_, 32, 8)

// CPL for 8 query heads: 8 with 4-bit codes (fewer key digit registers), else 16
#define KVQ_DECODE_TABLE_D128(BITS)                      \
    KVQ_DECODE_GROUPS_MHA(BITS, 128, 32)                 \
    KVQ_DECODE_GROUPS_MHA(BITS, 128, 16)                 \
    KVQ_DECODE_GROUPS_GQA(BITS, 128, 2, 16)              \
    KVQ_DECODE_GROUPS_GQA(BITS, 128, 4, 16)              \
    KVQ_DECODE_GROUPS_GQA(BITS, 128, 8, (BITS == 4 ? 8 : 16))

#define KVQ_DECODE_TABLE_D64(BITS)                       \
    KVQ_DECODE_GROUPS_MHA(BITS, 64, 16)                  \
    KVQ_DECODE_GROUPS_GQA(BITS, 64, 2, 16)               \
    KVQ_DECODE_GROUPS_GQA(BITS, 64, 4, 16)               \
    KVQ_DECODE_GROUPS_GQA(BITS, 64, 8, (BITS == 4 ? 8 : 16))

#define KVQ_DECODE_MF_CASE(BITS, D_, GQ_, TPG_, NVG_)                    \
    if (gqa == GQ_ && tpg == TPG_ && nvg == NVG_)                        \
        return reinterpret_cast<const void*>(&decode_kernel<BITS, D_, GQ_, 16, 64, TPG_, true, NVG_>);

#define KVQ_DECODE_MF_TPG(BITS, D_, GQ_, NVG_)   \
    KVQ_DECODE_MF_CASE(BITS, D_, GQ_, 1, NVG_)   \
    KVQ_DECODE_MF_CASE(BITS, D_, GQ_, 2, NVG_)   \
    KVQ_DECODE_MF_CASE(BITS, D_, GQ_, 4, NVG_)

#define KVQ_DECODE_MF_GQ(BITS, D_, NVG_)   \
    KVQ_DECODE_MF_TPG(BITS, D_, 2, NVG_)   \
    KVQ_DECODE_MF_TPG(BITS, D_, 4, NVG_)   \
    KVQ_DECODE_MF_TPG(BITS, D_, 8, NVG_)

// value groups of 64 channels or more: one or two per token at head_dim 128, one at 64
#define KVQ_DECODE_MF_TABLE_D128(BITS) KVQ_DECODE_MF_GQ(BITS, 128, 1) KVQ_DECODE_MF_GQ(BITS, 128, 2)
#define KVQ_DECODE_MF_TABLE_D64(BITS) KVQ_DECODE_MF_GQ(BITS, 64, 1)
// 8-bit codes run on the matrix cores only: one query head per kv head as well
#define KVQ_DECODE_MF8_TABLE_D128                                          \
    KVQ_DECODE_MF_TPG(8, 128, 1, 1) KVQ_DECODE_MF_TPG(8, 128, 1, 2) KVQ_DECODE_MF_TABLE_D128(8)
#define KVQ_DECODE_MF8_TABLE_D64 KVQ_DECODE_MF_TPG(8, 64, 1, 1) KVQ_DECODE_MF_TABLE_D64(8)

#define KVQ_DEFINE_MF8_KERNEL_PTR(D_)                                           \
    template <>                                                                 \
    const void* decode_mf_kernel_ptr<8, D_>(int gqa, int tpg, int nvg) {        \
        KVQ_DECODE_MF8_TABLE_D##D_                                              \
        return nullptr;                                                         \
    }

#define KVQ_DEFINE_MF_KERNEL_PTR(BITS, D_)                                           \
    template <>                                                                      \
    const void* decode_mf_kernel_ptr<BITS, D_>(int gqa, int tpg, int nvg) {          \
        KVQ_DECODE_MF_TABLE_D##D_(BITS)                                              \
        return nullptr;                                                              \
    }

#define KVQ_DECODE_SP_CASE(BITS, D_, GQ_, CPL_, TILE_, TPG_)                   \
    if (gqa == GQ_ && cpl == CPL_ && tile == TILE_ && tpg == TPG_)              \
        return reinterpret_cast<const void*>(&decode_kernel<BITS, D_, GQ_, CPL_, TILE_, TPG_, false, 1, true>);

// one value group per token on the four-lane, four-token map (D 128, 32 channels per lane, 64-token tiles)
#define KVQ_DECODE_SPW_CASE(BITS, TPG_)                                           \
    if (gqa == 1 && nvg == 1 && cpl == 32 && tile == 64 && tpg == TPG_)           \
        return reinterpret_cast<const void*>(&decode_kernel<BITS, 128, 1, 32, 64, TPG_, false, 1, true, true>);

#define KVQ_DECODE_SP_MHA(BITS, D_, CPL_)        \
    KVQ_DECODE_SP_CASE(BITS, D_, 1, CPL_, 32, 1) \
    KVQ_DECODE_SP_CASE(BITS, D_, 1, CPL_, 64, 1) \
    KVQ_DECODE_SP_CASE(BITS, D_, 1, CPL_, 64, 2) \
    KVQ_DECODE_SP_CASE(BITS, D_, 1, CPL_, 64, 4)

// several query heads per kv head: 32-token tiles, groups of 32 to 256 tokens
#define KVQ_DECODE_SP_GQA(BITS, D_, GQ_, CPL_)      \
    KVQ_DECODE_SP_CASE(BITS, D_, GQ_, CPL_, 32, 1)  \
    KVQ_DECODE_SP_CASE(BITS, D_, GQ_, CPL_, 32, 2)  \
    KVQ_DECODE_SP_CASE(BITS, D_, GQ_, CPL_, 32, 4)  \
    KVQ_DECODE_SP_CASE(BITS, D_, GQ_, CPL_, 32, 8)

#define KVQ_DECODE_SP_TABLE_D128(BITS)                                                          \
    KVQ_DECODE_SPW_CASE(BITS, 1) KVQ_DECODE_SPW_CASE(BITS, 2) KVQ_DECODE_SPW_CASE(BITS, 4)      \
    KVQ_DECODE_SP_MHA(BITS, 128, 32) KVQ_DECODE_SP_MHA(BITS, 128, 16)                           \
    KVQ_DECODE_SP_GQA(BITS, 128, 2, 16) KVQ_DECODE_SP_GQA(BITS, 128, 4, 16)                     \
    KVQ_DECODE_SP_GQA(BITS, 128, 8, (BITS == 4 ? 8 : 16))
#define KVQ_DECODE_SP_TABLE_D64(BITS)                                                           \
    KVQ_DECODE_SP_MHA(BITS, 64, 16) KVQ_DECODE_SP_GQA(BITS, 64, 2, 16) KVQ_DECODE_SP_GQA(BITS, 64, 4, 16) \
    KVQ_DECODE_SP_GQA(BITS, 64, 8, (BITS == 4 ? 8 : 16))

#define KVQ_DECODE_MFSP_CASE(BITS, GQ_, TPG_, NVG_)                      \
    if (gqa == GQ_ && tpg == TPG_ && nvg == NVG_)                        \
        return reinterpret_cast<const void*>(&decode_kernel<BITS, 128, GQ_, 16, 64, TPG_, true, NVG_, true>);
#define KVQ_DECODE_MFSP_TPG(BITS, GQ_, NVG_) \
    KVQ_DECODE_MFSP_CASE(BITS, GQ_, 1, NVG_) KVQ_DECODE_MFSP_CASE(BITS, GQ_, 2, NVG_) KVQ_DECODE_MFSP_CASE(BITS, GQ_, 4, NVG_)
#define KVQ_DEFINE_MFSP_KERNEL_PTR(BITS)                                                      \
    template <>                                                                               \
    const void* decode_mfsp_kernel_ptr<BITS>(int gqa, int tpg, int nvg) {                     \
        KVQ_DECODE_MFSP_TPG(BITS, 2, 1) KVQ_DECODE_MFSP_TPG(BITS, 4, 1) KVQ_DECODE_MFSP_TPG(BITS, 8, 1) \
        KVQ_DECODE_MFSP_TPG(BITS, 2, 2) KVQ_DECODE_MFSP_TPG(BITS, 4, 2) KVQ_DECODE_MFSP_TPG(BITS, 8, 2) \
        return nullptr;                                                                       \
    }

#define KVQ_DEFINE_SP_KERNEL_PTR(BITS, D_)                                      \
    template <>                                                                 \
    const void* decode_sp_kernel_ptr<BITS, D_>(int gqa, int cpl, int tile, int tpg, int nvg) { \
        KVQ_DECODE_SP_TABLE_D##D_(BITS)                                         \
        return nullptr;                                                         \
    }

// per-token keys: key groups of 64 or 128 tokens (one or two 64-token tiles)
#define KVQ_DECODE_KT_VALU(BITS, D_, CPL_, TPG_)                                         \
    if (!mf && gqa == 1 && cpl == CPL_ && tpg == TPG_)                                  \
        return reinterpret_cast<const void*>(                                          \
            &decode_kernel<BITS, D_, 1, CPL_, 64, TPG_, false, 1, false, false, true>);
#define KVQ_DECODE_KT_MF(BITS, D_, GQ_, TPG_, NVG_)                                      \
    if (mf && gqa == GQ_ && tpg == TPG_ && nvg == NVG_)                                 \
        return reinterpret_cast<const void*>(                                          \
            &decode_kernel<BITS, D_, GQ_, 16, 64, TPG_, true, NVG_, false, false, true>);
#define KVQ_DECODE_KT_MF_TPG(BITS, D_, GQ_, NVG_) \
    KVQ_DECODE_KT_MF(BITS, D_, GQ_, 1, NVG_) KVQ_DECODE_KT_MF(BITS, D_, GQ_, 2, NVG_)
#define KVQ_DECODE_KT_MF_GQ(BITS, D_, NVG_)                                             \
    KVQ_DECODE_KT_MF_TPG(BITS, D_, 2, NVG_) KVQ_DECODE_KT_MF_TPG(BITS, D_, 4, NVG_)     \
    KVQ_DECODE_KT_MF_TPG(BITS, D_, 8, NVG_)
#define KVQ_DECODE_KT_TABLE_D128(BITS)                                                  \
    KVQ_DECODE_KT_VALU(BITS, 128, 32, 1) KVQ_DECODE_KT_VALU(BITS, 128, 32, 2)           \
    KVQ_DECODE_KT_VALU(BITS, 128, 16, 1) KVQ_DECODE_KT_VALU(BITS, 128, 16, 2)           \
    KVQ_DECODE_KT_MF_GQ(BITS, 128, 1) KVQ_DECODE_KT_MF_GQ(BITS, 128, 2)
#define KVQ_DECODE_KT_TABLE_D64(BITS)                                                   \
    KVQ_DECODE_KT_VALU(BITS, 64, 16, 1) KVQ_DECODE_KT_VALU(BITS, 64, 16, 2) KVQ_DECODE_KT_MF_GQ(BITS, 64, 1)
// 8-bit codes: the matrix cores only, one query head per kv head as well
#define KVQ_DECODE_KT8_TABLE_D128                                                       \
    KVQ_DECODE_KT_MF_TPG(8, 128, 1, 1) KVQ_DECODE_KT_MF_TPG(8, 128, 1, 2)               \
    KVQ_DECODE_KT_MF_GQ(8, 128, 1) KVQ_DECODE_KT_MF_GQ(8, 128, 2)
#define KVQ_DECODE_KT8_TABLE_D64 KVQ_DECODE_KT_MF_TPG(8, 64, 1, 1) KVQ_DECODE_KT_MF_GQ(8, 64, 1)

#define KVQ_DEFINE_KT_KERNEL_PTR(BITS, D_, TABLE)                                       \
    template <>                                                                         \
    const void* decode_kt_kernel_ptr<BITS, D_>(int gqa, int cpl, int tpg, int nvg, bool mf) { \
        (void)cpl;                                                                      \
        TABLE                                                                           \
        return nullptr;                                                                 \
    }

#define KVQ_DEFINE_KERNEL_PTR(BITS, D_)                                               \
    template <>                                                                       \
    const void* decode_kernel_ptr<BITS, D_>(int gqa, int cpl, int tile, int tpg) {   \
        KVQ_DECODE_TABLE_D##D_(BITS)                                                  \
        return nullptr;                                                               \
    }

}  // namespace dec
}  // namespace kvq
