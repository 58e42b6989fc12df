// decode_impl.h -- split-token decode attention over the low-bit KV cache (gfx950).
//
// out = softmax(q K'^T * sm_scale) V' over sinks, quantized tokens and residual
// ("KV Cache的Int4量化：如何解决Attention Sink导致的量化精度崩塌问题", section 3;
// KIVI notes "LLM系列：KVCache量化1 KIVI…", section 1: the logits of the grouped
// part and of the residual are concatenated before one softmax).  Token order
// does not matter ("Resumo Técnico: LogQuant", Metodologia 4), so the tokens of
// every (sequence, kv head) slice are cut into splits that run in parallel; each
// split keeps an online-softmax state (running max m, sum l, unnormalised
// accumulator) and the last workgroup of the slice merges them (log-sum-exp).
//
// Arithmetic.  With k' = (c - z) s per channel (keys) and v' = (c - z) s per
// token group (values):
//   q . k' = sum_c (q_c s_c) (c - 8) - sum_c (q_c s_c) (z_c - 8)
//   sum_t p_t v'_tc = sum_t (p_t s_t) (c_tc - 8) - sum_t (p_t s_t) (z_t - 8)
// (the zero-point cross-term identity of "Atom…", section 三 "核心公式"; the 8 is
// the code bias for 4-bit codes, 0 for 2-bit codes).  The left sums are integer
// dot products of the packed codes with a fixed-point image of q_c s_c (per key
// group) or p_t s_t (per tile of tokens): the real operand is scaled by 2^k so its
// largest magnitude is below 2^18, rounded to an integer and split into five
// balanced base-16 digits in [-8, 7].  v_dot8c_i32_i4 multiplies eight signed
// nibbles of codes with eight digit nibbles and accumulates in int32, so one
// instruction does eight multiply-adds with no byte-to-float conversion; the
// digits are recombined by shifts (Horner) and scaled back by 2^-k in fp32.  The
// rounding of the fixed-point image is the only approximation (relative 2^-19 of
// the group's largest |q_c s_c| or of the tile's largest p_t s_t).
//
// Mapping on CDNA4 (wave64), one workgroup = 4 waves = one split:
//   - a slice's quantized part is a stream of key-group records (key scales and
//     zeros, key code rows, value code blocks, value scales and zeros); wave w of
//     the split streams groups w, w+4, ... tile by tile through a ring of
//     tiles, the next ones in flight while one is processed;
//   - keys: a token row is spread over LPT = D / CPL lanes (CPL codes each), so a
//     wave scores TPW = 64 / LPT tokens per load; the per-lane integer partials
//     are summed over the LPT lanes with DPP;
//   - values: dword (block, channel) of the value codes holds one channel of TB
//     consecutive tokens; a lane owns D/32 channels of one block, so its value
//     dot products run along tokens;
//   - the folded query's digits go through LDS as bytes that already pair the
//     channels of a code nibble dword (the writer takes the partner channel's
//     digits from a neighbouring lane), so a lane reads its digit dwords whole;
//   - the softmax weights' digits move between the two mappings through LDS as
//     bytes that pair the tokens of a value code nibble dword (a key slot scores
//     whole token pairs), so a value lane reads its digit dwords whole;
//   - all five digits of an integer come from one add and one xor (n + 0x88888
//     holds each digit + 8 in its nibble);
//   - issue priority falls as a wave's stream advances, so of two workgroups
//     sharing a CU the one with less done is served first;
//   - the running max is wave-uniform and updated once per tile;
//   - sinks and residual tokens (full precision) are spread over the splits and
//     scored with fp32 FMAs through the same state;
//   - all GQ query heads that share a kv head run in the same workgroup, so each
//     KV byte is read from HBM once.
#pragma once

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace dec {

struct DecArgs {
    const uint8_t* rec;  // key-group records
    const char* ksink;
    const char* vsink;
    const char* kres;
    const char* vres;
    const char* knew;    // fused append: newest token's K, V rows [BH][D], or null
    const char* vnew;
    const void* q;
    float* out;
    float* lse;
    float* part_acc;     // [BH][nsplit_cap][GQ][D]
    float* part_ml;      // [BH][nsplit_cap][GQ][2]
    unsigned* counters;  // [BH] slice counters, then the group counters
    int64_t ng_cap;
    int rec_bytes, rec_kcodes, rec_vcodes, rec_vmeta;
    int rec_kov, rec_koi, rec_vov, rec_voi;  // outlier fields of dense-and-sparse records
    int dtype;  // storage dtype of q, sinks and residual (DT_*)
    int Hkv, S, R, Qf, nS, nfp, G, GV, nvg, gps, ngroups, nsplit, nsplit_cap;
    // Paged records (table non-null): rec is the page pool (pool_bytes < 4 GiB),
    // page table int32 [B][max_pages], 2^lp key groups per page, page_bytes each.
    const int* table;
    int lp, max_pages, pool_pages;
    uint32_t page_bytes, pool_bytes;
    float qscale;  // sm_scale * log2(e)
    // Sequences of different lengths: sequence b holds base_len[b] + len_delta
    // tokens, and nS, nfp, ngroups above are replaced by its own; null otherwise.
    const int* base_len;
    int len_delta;
    // Two-level split combine: splits in groups of cgs (cgs >= nsplit: one level);
    // group partials [BH][cgroups_cap][GQ][D] and [BH][cgroups_cap][GQ][2], group
    // counters [BH][cgroups_cap] after the slice counters.
    float* grp_acc;
    float* grp_ml;
    int cgs, cgroups_cap;
    // Split weights: splits below s1 take gps key groups, the others gps2; the grid
    // is then split-major (split_major = 1).
    int s1, gps2, split_major;
};

constexpr int kLimbs = 5;

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------
// Every control used here (quad permutes, row mirrors) reads a valid lane for
// every lane, so bound_ctrl only lets the move fold into the consuming operation.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Lane l's value (l wave-uniform), read into a scalar register.
__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Whole-wave sum and max when every lane of each 16-lane row holds its row's
// result r0..r3: row_bcast:15 combines row 0's result into row 1 and row 2's into
// row 3, row_bcast:31 then combines lane 31 (rows 0 and 1) into row 3, and lane
// 63's total, (r3 + r2) + (r1 + r0), is read as a scalar, so every lane gets the
// same bits (the same as any order of the two pairs).  Full exec mask required.
// Each step is one DPP add or max whose row mask leaves the other rows' values in
// place (built from an update_dpp and an add, the compiler emits a copy, a DPP move
// and the add).  The compiler does not see DPP inside the asm, so the asm keeps
// the wait states itself: two before each DPP read of a VGPR just written by a
// VALU instruction, and one before a v_readlane of it.
__device__ __forceinline__ float rows_sum(float v) {
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0x8 bank_mask:0xf\n\t"
        "s_nop 0"
        : "+v"(v));
    return lane_value(v, 63);
}
__device__ __forceinline__ float rows_max(float v) {
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0x8 bank_mask:0xf\n\t"
        "s_nop 0"
        : "+v"(v));
    return lane_value(v, 63);
}

// Sum over aligned groups of N consecutive lanes; every lane of a group gets the
// same (bitwise identical) sum.  N = 64 needs the full exec mask.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (N >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (N == 32) v += __shfl_xor(v, 16);
    if constexpr (N == 64) v = rows_sum(v);
    return v;
}

// Max over aligned groups of N consecutive lanes (same pattern as group_sum).
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
    if constexpr (N == 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (N == 64) v = rows_max(v);
    return v;
}

// Max over the slots of a wave when every group of LPT lanes holds one value:
// reduces lanes LPT apart (values are equal inside a group).  Full exec mask.
template <int LPT>
__device__ __forceinline__ float slots_max(float v) {
    if constexpr (LPT == 1) return group_max<64>(v);
    else if constexpr (LPT == 2) { v = fmaxf(v, dpp<0x4E>(v)); }
    if constexpr (LPT <= 4) v = fmaxf(v, dpp<0x141>(v));
    if constexpr (LPT <= 8) v = fmaxf(v, dpp<0x140>(v));
    return rows_max(v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// True when the predicate holds on any active lane; the result is a scalar, so a
// branch on it is a scalar branch.  Used for predicates that are wave-uniform by
// construction but that the compiler cannot prove uniform.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// f(std::integral_constant<int, I>()) for I = 0 .. N - 1, unrolled at compile time.
template <int I, int N>
struct StaticFor {
    template <typename F>
    __device__ __forceinline__ static void run(F& f) {
        if constexpr (I < N) {
            f(std::integral_constant<int, I>());
            StaticFor<I + 1, N>::run(f);
        }
    }
};

// A kernel-argument pointer as an opaque wave-uniform value.  Selects between
// such values stay selects; selects between the argument fields themselves may
// be rewritten into a per-lane load of the chosen field.
__device__ __forceinline__ const char* arg_ptr(const char* p) {
    typedef __attribute__((address_space(1))) const char gchar;
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    // a global-memory pointer, so that accesses through it stay global accesses
    return (const char*)reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}

// Buffer loads: a buffer resource (base address and size in scalar registers), a
// per-lane byte offset, and a wave-uniform byte offset in a scalar register.  The
// per-lane offsets of a tile stream stay fixed and only the scalar offset moves,
// so a tile load costs no vector address arithmetic.  Third descriptor dword for
// gfx9-family raw buffers (32-bit data format, no swizzle, no stride).
constexpr int kBufferWord3 = 0x00020000;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
// Byte offset, inside the records' buffer resource, of key group g0 + kWaves j
// (a wave's j-th group, at most gmax): page_off of lane (g >> lp) - p_first plus
// the group's place in its page.  Paged records: lane i of page_off holds the
// offset of page p_first + i of this slice's split (at most 64 pages), always a
// page of the pool.  Contiguous records are one page over the slice's own
// resource (lp = 31, page_off = 0, gmax = its last record).  Every offset so
// lies inside the resource, for the groups a wave loads beyond its own too.
struct GroupAddr {
    int g0, gmax, lp, p_first;
    uint32_t mask, rec_bytes, page_off;
    __device__ __forceinline__ uint32_t at(int j) const {
        const int g = min(g0 + kWaves * j, gmax);
        const uint32_t po = (uint32_t)__builtin_amdgcn_readlane((int)page_off, (g >> lp) - p_first);
        return po + ((uint32_t)g & mask) * rec_bytes;
    }
};

template <int N>
struct UVec {
    typedef uint32_t T __attribute__((ext_vector_type(N)));
};
template <>
struct UVec<1> {
    typedef uint32_t T;
};
template <int N>
__device__ __forceinline__ typename UVec<N>::T bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (N == 1) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    else if constexpr (N == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    else {
        static_assert(N == 4, "1, 2 or 4 dwords");
        return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    }
}
// Element i of a dword vector (or the dword itself).
template <typename T>
__device__ __forceinline__ uint32_t elem(const T& v, int i) {
    if constexpr (sizeof(T) == 4) return v;
    else return v[i];
}
// Hands a whole register tuple to the code that follows.  Without it, the
// vectors a tile buffer holds are split into single dwords, and such buffers
// carried around a loop are not kept in the registers their loads write (the
// back edge then copies them, waiting for the loads in flight).
template <typename T>
__device__ __forceinline__ T whole(T v) {
    asm("" : "+v"(v));
    return v;
}

// Orders this wave's LDS writes before its following LDS reads (one wave only).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// device-scope store / load of split partials exchanged between workgroups
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two adjacent floats (8-byte aligned) with one device-scope load.
__device__ __forceinline__ float2 fetch2(const float* p) {
    const unsigned long long v = __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<float*>(p)),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return float2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}

__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
// The same with a zero accumulator, as the three-operand form with an inline 0
// (the builtin with c = 0 becomes a register cleared to 0 and the accumulating form).
__device__ __forceinline__ int dot8_0(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Fixed-point scale for values of magnitude <= maxabs: mul = 2^(18-E), inv = 2^(E-18)
// with maxabs < 2^E, so |rint(x * mul)| <= 2^18 fits five balanced hex digits.
struct FixScale {
    float mul, inv;
};
__device__ __forceinline__ FixScale fix_scale(float maxabs) {
    int E = (int)((__float_as_uint(maxabs) >> 23) & 0xFFu) - 126;
    E = E < -100 ? -100 : E;
    FixScale f;
    f.mul = __uint_as_float((uint32_t)(127 + 18 - E) << 23);
    f.inv = __uint_as_float((uint32_t)(127 - 18 + E) << 23);
    return f;
}

// (a & m) | (b & ~m) in one instruction (the compiler emits an and and an and-or)
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
    return r;
}

// Pair bytes of two digit words x (low nibbles) and y (high nibbles), all five
// limbs as two's-complement nibbles: limbs 0, 2, 4 in bytes 0, 1, 2 of ev, limbs
// 1, 3 in bytes 0, 1 of od.
__device__ __forceinline__ void pair_bytes(uint32_t x, uint32_t y, uint32_t& ev, uint32_t& od) {
    ev = bfi(0x0F0F0Fu, x, y << 4);
    od = bfi(0x0F0F0Fu, x >> 4, y);
}

// Stores limb li's pair byte of each of N pair words (pair_bytes) as N consecutive
// bytes at dst + li * stride.
template <int N>
__device__ __forceinline__ void store_limb_bytes(uint8_t* dst, int stride, const uint32_t (&ev)[N],
                                                 const uint32_t (&od)[N]) {
    if constexpr (N == 1) {
        dst[0] = (uint8_t)ev[0];
        dst[2 * stride] = (uint8_t)(ev[0] >> 8);
        dst[4 * stride] = (uint8_t)(ev[0] >> 16);
        dst[stride] = (uint8_t)od[0];
        dst[3 * stride] = (uint8_t)(od[0] >> 8);
    } else if constexpr (N == 2) {
        // bytes (k of word 0, k of word 1) for k = 0, 1 (limbs 0 and 2, or 1 and 3), and k = 2
        const uint32_t e02 = __builtin_amdgcn_perm(ev[1], ev[0], 0x05010400u);
        const uint32_t e4 = __builtin_amdgcn_perm(ev[1], ev[0], 0x0C0C0602u);
        const uint32_t o13 = __builtin_amdgcn_perm(od[1], od[0], 0x05010400u);
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)e02;
        *reinterpret_cast<uint16_t*>(dst + 2 * stride) = (uint16_t)(e02 >> 16);
        *reinterpret_cast<uint16_t*>(dst + 4 * stride) = (uint16_t)e4;
        *reinterpret_cast<uint16_t*>(dst + stride) = (uint16_t)o13;
        *reinterpret_cast<uint16_t*>(dst + 3 * stride) = (uint16_t)(o13 >> 16);
    } else {
        static_assert(N == 4, "1, 2 or 4 bytes per limb");
#pragma unroll
        for (int li = 0; li < kLimbs; ++li) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < N; ++i) w |= ((((li & 1) ? od[i] : ev[i]) >> (8 * (li >> 1))) & 0xFFu) << (8 * i);
            *reinterpret_cast<uint32_t*>(dst + li * stride) = w;
        }
    }
}

// The five balanced base-16 digits of U integers (|n| <= 2^18), paired: byte i of
// limb li's run (runs `stride` bytes apart) holds digit li of n[i] in its low
// nibble and that of n[i + U / 2] in its high nibble, as two's-complement nibbles.
// n + 0x88888 holds digit + 8 in every nibble (the balanced digits of |n| <= 2^18
// are the offset digits of n + 0x88888), and the exclusive or with 0x88888 turns
// each nibble into its digit's 4-bit form, so one add and one xor give all five.
template <int U>
__device__ __forceinline__ void store_pair_digits(uint8_t* dst, int stride, const int (&n)[U]) {
    constexpr int UH = U / 2;
    uint32_t ev[UH], od[UH];
#pragma unroll
    for (int i = 0; i < UH; ++i)
        pair_bytes((uint32_t)(n[i] + 0x88888) ^ 0x88888u, (uint32_t)(n[i + UH] + 0x88888) ^ 0x88888u, ev[i], od[i]);
    store_limb_bytes<UH>(dst, stride, ev, od);
}

__device__ __forceinline__ uint32_t lds32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// Key digit bytes of the VALU stream, paired.  A nibble dword of codes holds the
// codes of channel pairs (c, c + P), c a "lo" channel (c mod 2P < P): P = 4 for
// 4-bit codes, 8 for 2-bit codes.  Limb li of a head's folded query is stored as
// D/2 bytes, one per pair: the digit of c in the low nibble, that of c + P in the
// high one, at byte (c / 2P) P + c mod 2P.  A lane's digit dwords of one limb (its
// CPL channels, a multiple of 2P) are then consecutive, read without combining.
// The writer lane of KM channels c.. (c lo) takes the digits of c + P.. from lane
// + P / KM (a DPP row shift within the row of 16 lanes); the lanes of hi channels
// write the same pattern into a second, unread area of the same size.
template <int KM, int P>
__device__ __forceinline__ void store_key_digits(uint8_t* lo_base, uint8_t* hi_base, int stride, int lane,
                                                 const int (&n)[KM]) {
    static_assert(KM == 1 || KM == 2, "one or two fold channels per lane");
    constexpr int KPL = P / KM;                  // lanes from the owner of c to that of c + P
    static_assert(KPL >= 1 && 2 * KPL <= 16, "pair partner within the lane's row");
    // All five digits of channel c + j as two's-complement nibbles (the add and
    // xor of store_pair_digits), those of c + P + j from the partner lane, and
    // their pair bytes: limbs 0, 2, 4 in bytes 0, 1, 2 of ev, limbs 1, 3 of od.
    uint32_t ev[KM], od[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        const uint32_t x = (uint32_t)(n[j] + 0x88888) ^ 0x88888u;
        pair_bytes(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x100 + KPL, 0xF, 0xF, true), ev[j], od[j]);
    }
    const int c = KM * lane;
    const bool lo = c % (2 * P) < P;
    const int cl = lo ? c : c - P;
    store_limb_bytes<KM>((lo ? lo_base : hi_base) + (cl / (2 * P)) * P + cl % (2 * P), stride, ev, od);
}

// nw dwords from p (aligned to the largest load used): 16-byte loads where they
// fit, then 8 and 4.
__device__ __forceinline__ void load_dwords(const char* p, uint32_t* w, int nw) {
    int i = 0;
    for (; i + 4 <= nw; i += 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(p + 4 * i);
        w[i] = x.x, w[i + 1] = x.y, w[i + 2] = x.z, w[i + 3] = x.w;
    }
    for (; i + 2 <= nw; i += 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(p + 4 * i);
        w[i] = x.x, w[i + 1] = x.y;
    }
    for (; i < nw; ++i) w[i] = *reinterpret_cast<const uint32_t*>(p + 4 * i);
}

// Element i of packed storage words as fp32.
template <int DT>
__device__ __forceinline__ float packed_f32(const uint32_t* w, int i) {
    if constexpr (DT == DT_F32) return __uint_as_float(w[i]);
    else if constexpr (DT == DT_BF16) return __uint_as_float((w[i >> 1] >> (16 * (i & 1))) << 16);
    else return f16_to_f32((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
}

// ---------------------------------------------------------------------------
// Quantized stream on the matrix cores, for several query heads per kv head.
//
// With GQ query heads sharing a kv head, the key and value dot products of a
// tile are small dense matrix products: scores [heads x tokens] = Q' [heads x
// channels] . K^T, and outputs [heads x channels] += W [heads x tokens] . V.  They
// run on v_mfma_i32_16x16x64_i8 in exact integer arithmetic.  The fixed-point
// operand (the folded query q_c s_c of a key group, or the weights p_t s_t of a
// tile; |n| <= 2^18 as in the VALU path) is split into three balanced base-256
// digits, and each (query head, digit) pair is one row of the 16-row A operand
// (rows 4 h + digit; row 4 h + 3 and absent heads are zero).  The codes are the B
// operand: 4- and 2-bit codes unpacked to unsigned bytes, 8-bit fields (int8
// code - 128) as loaded.  The digits are recombined by shifts (Horner) in int32
// for 4- and 2-bit codes (|sum_c n_c u_c| <= 2^18 * 15 * 128 < 2^31), in fp32 for
// 8-bit codes.  Zero points enter through sum_c (q_c s_c) (z_c - o) and
// sum_t (p_t s_t) (z_t - o) in fp32 (o = 128 for 8-bit fields, else 0), as in
// the VALU path.  One query head per kv head is the case GQ = 1 (8-bit codes).
//
// Operand layout of the instruction (lane l, byte e of its 16 bytes): A row l % 16,
// k = 16 (l / 16) + e; B column l % 16, same k; result column l % 16, rows
// 4 (l / 16) .. + 3, so lane l holds all digit rows of head l / 16 of its block.
//   keys:   16 tokens per product (column j = token), k = channel: lane l reads
//           the D/4 channels (D/4) (l / 16) .. of token l % 16 with one load;
//   values: 64 tokens per product (k = token 16 (l / 16) + e), 16 channels per
//           product: product n holds channels 64 (n / 4) + 4 j + n % 4 (j = column),
//           so the 16 columns of a product share one value group (G_V >= 64) and a
//           lane loads four adjacent channels with one 16-byte load.
// A tile is 64 tokens of one key group; a ring of tiles streams the wave's groups
// as in the VALU path.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_i8(const i32x4& a, const i32x4& b, const i32x4& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// the three balanced base-256 digits of n (|n| <= 2^18) as int8 bytes 0, 1, 2
__device__ __forceinline__ uint32_t digits256(int n) { return ((uint32_t)(n + 32896) ^ 0x8080u); }

// exact recombination of digit rows 0..2 of a product (row 3 is zero)
__device__ __forceinline__ int horner256(const i32x4& r) { return (r[2] * 256 + r[1]) * 256 + r[0]; }

// SP: dense-and-sparse records.  The outliers' differences from their codes'
// values go through per-wave LDS tables as on the VALU stream: key terms onto the
// scores of the group's tokens (once per group), value terms onto the channels of
// the tile's outputs.  A lane owns one (head, token) pair of each score product
// and one (head, channel) pair of each output accumulator.
// Streams that run two waves per SIMD (two workgroups per CU) with a ring of two
// tiles: dense-and-sparse ones on the VALU and 2-bit matrix-core ones, with at
// most four query heads per kv head.  They fit in 256 registers (a few spill
// outside the loop), and the second wave hides the per-tile latency of the first
// (reductions, LDS round trips, the outlier tables' atomics), which bounds these
// streams rather than HBM.  Plain 4- and 8-bit streams, the plain VALU stream and
// the 4-bit dense-and-sparse matrix-core stream are HBM-bound and keep one wave
// per SIMD with a ring of four tiles, which keeps more bytes in flight (measured
// on the GQA outlier workload: 126 against 129 us with two waves); eight query
// heads per kv head would spill at 256 registers.
__host__ __device__ constexpr bool two_waves(bool mf, int bits, int gq, bool sp) {
    return gq <= 4 && ((mf && bits == 2) || (sp && !mf));
}

// KT: per-token keys (one scale and zero point per token over its D channels):
// the query's digit rows are folded once per wave, not per key group, and each
// score takes its token's scale s_t and zero z_t after the product:
//   q . k'_t = s_t (sum_c q_c u_tc - (z_t - o) sum_c q_c)
// with sum_c q_c taken over the query's fixed-point image.
template <int BITS, int D, int GQ, int TPG, int NVG, bool SP = false, bool KT = false>
struct MStream {
    static constexpr int TM = 64;               // tokens per tile
    static constexpr int NSB = TM / 16;         // key products per tile and row block
    static constexpr int RBK = (GQ + 3) / 4;    // 16-row blocks (four heads each)
    static constexpr int NKK = D / 64;          // key products per 16 tokens (64 channels each)
    static constexpr int NVB = D / 64;          // 64-channel blocks of the values
    static constexpr int NVM = D / 16;          // value products per row block
    static constexpr int TB = 32 / BITS;        // tokens per value dword
    static constexpr int VBB = 16 / TB;         // value dwords per lane, channel and tile
    static constexpr int RB = D * BITS / 8;     // key row bytes
    static constexpr int KLW = RB / 16;         // key dwords per lane and token
    static constexpr int KLD = KLW > 4 ? 4 : KLW;  // dwords per key load
    static constexpr int KLN = KLW / KLD;          // key loads per lane and token
    // 8-bit fields are int8 code - 128 (used as stored); 4- and 2-bit codes are
    // unpacked to unsigned bytes
    static constexpr float ZOFF = BITS == 8 ? 128.0f : 0.0f;
    static constexpr int KM = D / 64;           // fold channels per lane
    static constexpr int VCPL = D / 32;
    static constexpr int AK_BYTES = RBK * NKK * 1024;
    static constexpr int AV_BYTES = NVG * RBK * 1024;
    // Ring of NRM tile buffers, NRM - 1 in flight while one is processed.  (Six
    // buffers measured slower: more register traffic per tile.)
    static constexpr int NRM = two_waves(true, BITS, GQ, SP) ? 2 : 4;
    static constexpr int BODY = TPG > NRM ? TPG : NRM;  // tiles per loop iteration
    static constexpr int GB = BODY / TPG;               // key groups per loop iteration
    static __host__ __device__ constexpr int lds_bytes() { return AK_BYTES + 2 * AV_BYTES; }

    struct Tile {
        typename UVec<KLD>::T k[NSB][KLN];
        u32x4 v[NVB][VBB];
        typename UVec<2 * NVG>::T vm[NSB];  // (scale, zero) of each value group of token 16 sb + l % 16
        typename UVec<KM>::T ks, kz;
        typename UVec<2>::T km[NSB];  // KT: (scale, zero) of token 16 sb + l % 16
        // SP only: key outliers of the KM fold channels (values; dword of u16 fields),
        // value outliers of token 16 sb + l % 16 (values; dword of its groups' u16 fields)
        typename UVec<KM>::T kov;
        uint32_t koi;
        typename UVec<NVG>::T vov[NSB];
        uint32_t voi[NSB];
    };
    static constexpr int GT = TM * TPG;  // tokens per key group
    int* kc;       // SP: key outlier terms [GQ][GT], fixed point of 2^-k
    int* vc;       // SP: value outlier terms [GQ][D], fixed point
    float kc_inv;  // SP: 2^-k of the key group's terms
    uint32_t kov_off, koi_off, vov_off, voi_off;
    int koi_shift, voi_shift;

    __amdgpu_buffer_rsrc_t rs;
    GroupAddr ga;
    int last_group, lane;
    uint32_t k_off, v_off, vm_off, km_off, kt_off;
    uint8_t* ak_lds;  // [RBK][NKK][16 rows][64 bytes]
    uint8_t* av_lds;  // [2][NVG][RBK][16 rows][64 bytes]
    Tile t[NRM];
    i32x4 ak[RBK][NKK];
    float kinv_l[RBK], kbias_l[RBK];
    float kqs_l[RBK];  // KT: sum over channels of the lane's head's folded query (fixed-point image)
    float m_l[RBK], l2[RBK], z2[RBK][NVG], acc2[RBK][NVM];

    __device__ __forceinline__ void init(const DecArgs& a, __amdgpu_buffer_rsrc_t rsrc, const GroupAddr& addr,
                                         int n_my_groups, int ln, uint8_t* lds) {
        lane = ln;
        rs = rsrc;
        ga = addr;
        last_group = n_my_groups - 1;
        const int j = lane & 15, kb = lane >> 4;
        k_off = (uint32_t)a.rec_kcodes + j * RB + kb * (KLW * 4);
        v_off = (uint32_t)a.rec_vcodes + (kb * VBB * D + 4 * j) * 4;
        vm_off = (uint32_t)a.rec_vmeta + j * NVG * 8;
        km_off = KM * lane * 4;
        kt_off = j * 8;
        ak_lds = lds;
        av_lds = lds + AK_BYTES;
        kc = reinterpret_cast<int*>(lds + lds_bytes());
        vc = kc + GQ * GT;
        kov_off = (uint32_t)a.rec_kov + KM * lane * 4;
        koi_off = (uint32_t)a.rec_koi + ((KM * lane * 2) & ~3);
        koi_shift = KM == 1 ? 16 * (lane & 1) : 0;
        vov_off = (uint32_t)a.rec_vov + j * NVG * 4;
        voi_off = (uint32_t)a.rec_voi + ((j * NVG * 2) & ~3);
        voi_shift = NVG == 1 ? 16 * (j & 1) : 0;
        // padding rows (digit row 3 of every head, absent heads) stay zero
        for (int i = lane * 16; i < lds_bytes(); i += 64 * 16) *reinterpret_cast<u32x4*>(lds + i) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb) {
            m_l[rb] = -INFINITY;
            l2[rb] = 0.0f;
#pragma unroll
            for (int g = 0; g < NVG; ++g) z2[rb][g] = 0.0f;
#pragma unroll
            for (int n = 0; n < NVM; ++n) acc2[rb][n] = 0.0f;
        }
    }

    // Tile `tig` of the wave's key group j (groups past the last reload the last).
    __device__ __forceinline__ void load(Tile& tt, int j, int tig, bool kmeta) {
        const uint32_t grp = ga.at(min(j, max(last_group, 0)));
        const int t0 = tig * TM;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int ln = 0; ln < KLN; ++ln) tt.k[sb][ln] = bload<KLD>(rs, k_off + 16 * ln, grp + (t0 + 16 * sb) * RB);
#pragma unroll
        for (int m = 0; m < NVB; ++m)
#pragma unroll
            for (int bb = 0; bb < VBB; ++bb)
                tt.v[m][bb] = bload<4>(rs, v_off, grp + ((t0 / TB + bb) * D + 64 * m) * 4);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) tt.vm[sb] = bload<2 * NVG>(rs, vm_off, grp + (t0 + 16 * sb) * NVG * 8);
        if constexpr (KT) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) tt.km[sb] = bload<2>(rs, kt_off, grp + (t0 + 16 * sb) * 8);
        }
        if (!KT && kmeta) {  // constant at every call site
            tt.ks = bload<KM>(rs, km_off, grp);
            tt.kz = bload<KM>(rs, km_off + D * 4, grp);
            if constexpr (SP) {
                tt.kov = bload<KM>(rs, kov_off, grp);
                tt.koi = bload<1>(rs, koi_off, grp);
            }
        }
        if constexpr (SP) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                tt.vov[sb] = bload<NVG>(rs, vov_off, grp + (t0 + 16 * sb) * NVG * 4);
                tt.voi[sb] = bload<1>(rs, voi_off, grp + (t0 + 16 * sb) * NVG * 2);
            }
        }
    }

    // the first NRM - 1 tiles, in ring order
    __device__ __forceinline__ void start() {
        auto first = [&](auto ic) __attribute__((always_inline)) {
            constexpr int I = decltype(ic)::value;
            load(t[I], I / TPG, I % TPG, I % TPG == 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        StaticFor<0, NRM - 1>::run(first);
    }

    // Key group fold: digit rows of rint(q_c s_c 2^k) into LDS in product order,
    // then this lane's A operands; per-lane 2^-k and zero-point term of its head.
    __device__ __forceinline__ void fold(const Tile& cur, const float (&qv)[GQ][KM]) {
        const auto ks = whole(cur.ks), kz = whole(cur.kz);
        float qt[GQ][KM], mx[GQ], bp[GQ], kinv[GQ], kbias[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            mx[h] = 0.0f;
            bp[h] = 0.0f;
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                qt[h][j] = qv[h][j] * __uint_as_float(elem(ks, j));
                mx[h] = fmaxf(mx[h], fabsf(qt[h][j]));
                bp[h] = fmaf(qt[h][j], __uint_as_float(elem(kz, j)) - ZOFF, bp[h]);
            }
        }
        // One fixed-point scale for the group's query heads, from their largest
        // |q_c s_c|: one whole-wave reduction instead of one per head.
        float mxa = mx[0];
#pragma unroll
        for (int h = 1; h < GQ; ++h) mxa = fmaxf(mxa, mx[h]);
        const FixScale fs = fix_scale(group_max<64>(mxa));
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            kinv[h] = fs.inv;
            kbias[h] = group_sum<64>(bp[h]);
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                const int c = KM * lane + j;
                const int kb = c / (D / 4), kk = (c % (D / 4)) / 16, e = c % 16;
                uint8_t* dst = ak_lds + ((h / 4 * NKK + kk) * 16 + 4 * (h % 4)) * 64 + kb * 16 + e;
                const uint32_t d = digits256((int)rintf(qt[h][j] * fs.mul));
                dst[0] = (uint8_t)d;
                dst[64] = (uint8_t)(d >> 8);
                dst[128] = (uint8_t)(d >> 16);
            }
        }
        if constexpr (SP) {
            // key outliers: q_c (x_c - (u_c - z_c) s_c) onto the score of token t_c, added
            // in fixed point (LDS integer atomics; float ones run far slower): each term
            // below 2^23 units of the group's largest, so the at most D terms of one
            // token stay within int32
            const auto kov = whole(cur.kov);
            float kt[KM][GQ], kmx = 0.0f;
            int tk[KM];
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                const uint32_t e = (cur.koi >> (KM == 1 ? koi_shift : 16 * j)) & 0xFFFFu;
                const float delta = __uint_as_float(elem(kov, j)) -
                                    ((float)(e >> 8) - __uint_as_float(elem(kz, j))) * __uint_as_float(elem(ks, j));
                tk[j] = (int)(e & 0xFFu);
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    kt[j][h] = qv[h][j] * delta;
                    kmx = fmaxf(kmx, fabsf(kt[j][h]));
                }
            }
            const FixScale fs = fix_scale(group_max<64>(kmx));
            const float kmul = fs.mul * 32.0f;
            kc_inv = fs.inv * (1.0f / 32.0f);
#pragma unroll
            for (int h = 0; h < GQ; ++h)
#pragma unroll
                for (int i = 0; i < (GT + 63) / 64; ++i) kc[h * GT + ((i * 64 + lane) & (GT - 1))] = 0;
#pragma unroll
            for (int j = 0; j < KM; ++j)
#pragma unroll
                for (int h = 0; h < GQ; ++h) atomicAdd(&kc[h * GT + tk[j]], (int)rintf(kt[j][h] * kmul));
        }
        wave_lds_sync();
        const int hs = lane >> 4;
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                ak[rb][kk] = *reinterpret_cast<const i32x4*>(ak_lds + ((rb * NKK + kk) * 16 + (lane & 15)) * 64 + hs * 16);
            float ki = 0.0f, kbi = 0.0f;
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
                if (4 * rb + hh < GQ) {
                    ki = hs == hh ? kinv[4 * rb + hh] : ki;
                    kbi = hs == hh ? kbias[4 * rb + hh] : kbi;
                }
            kinv_l[rb] = ki;
            kbias_l[rb] = kbi;
        }
    }

    // Per-token keys: the query's digit rows (no key scale folded in), once per
    // wave; per lane 2^-k and the image's channel sum of its head.
    __device__ __forceinline__ void fold_kt(const float (&qv)[GQ][KM]) {
        float kinv[GQ], kqs[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            float mx = 0.0f;
#pragma unroll
            for (int j = 0; j < KM; ++j) mx = fmaxf(mx, fabsf(qv[h][j]));
            const FixScale fs = fix_scale(group_max<64>(mx));
            kinv[h] = fs.inv;
            float nsum = 0.0f;
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                const int c = KM * lane + j;
                const int kb = c / (D / 4), kk = (c % (D / 4)) / 16, e = c % 16;
                uint8_t* dst = ak_lds + ((h / 4 * NKK + kk) * 16 + 4 * (h % 4)) * 64 + kb * 16 + e;
                const int n = (int)rintf(qv[h][j] * fs.mul);
                const uint32_t d = digits256(n);
                dst[0] = (uint8_t)d;
                dst[64] = (uint8_t)(d >> 8);
                dst[128] = (uint8_t)(d >> 16);
                nsum += (float)n;
            }
            kqs[h] = group_sum<64>(nsum) * fs.inv;
        }
        wave_lds_sync();
        const int hs = lane >> 4;
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                ak[rb][kk] = *reinterpret_cast<const i32x4*>(ak_lds + ((rb * NKK + kk) * 16 + (lane & 15)) * 64 + hs * 16);
            float ki = 0.0f, kq = 0.0f;
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
                if (4 * rb + hh < GQ) {
                    ki = hs == hh ? kinv[4 * rb + hh] : ki;
                    kq = hs == hh ? kqs[4 * rb + hh] : kq;
                }
            kinv_l[rb] = ki;
            kqs_l[rb] = kq;
            kbias_l[rb] = 0.0f;
        }
    }

    // Digit rows of one product back to the integer sum: in int32 (Horner) for
    // 4- and 2-bit codes, whose totals stay below 2^31; in fp32 for 8-bit codes
    // (each row sum is exact in fp32, the total may exceed 2^31).
    __device__ __forceinline__ static float combine(const i32x4& r) {
        if constexpr (BITS == 8) return fmaf((float)r[2], 65536.0f, fmaf((float)r[1], 256.0f, (float)r[0]));
        else return (float)horner256(r);
    }

    // unsigned code bytes of four 4-bit codes (two dwords of 8) or of sixteen
    // 2-bit codes (one dword), in item order
    __device__ __forceinline__ static i32x4 unpack(uint32_t w0, uint32_t w1) {
        if constexpr (BITS == 4) {
            w0 ^= 0x88888888u;
            w1 ^= 0x88888888u;
            return i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
                         (int)((w1 >> 4) & 0x0F0F0F0Fu)};
        } else {
            return i32x4{(int)(w0 & 0x03030303u), (int)((w0 >> 2) & 0x03030303u), (int)((w0 >> 4) & 0x03030303u),
                         (int)((w0 >> 6) & 0x03030303u)};
        }
    }

    // One tile: scores on the matrix cores, softmax update, weight digits through
    // LDS (buffer `buf` of two), value products folded into fp32.
    __device__ __forceinline__ void process(const Tile& cur, int buf, int tig) {
        const i32x4 zero = {0, 0, 0, 0};
        float sc[RBK][NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            i32x4 bk[NKK];
            if constexpr (BITS == 8) {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) bk[kk] = __builtin_bit_cast(i32x4, whole(cur.k[sb][kk]));
            } else {
                const auto kw = whole(cur.k[sb][0]);
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    if constexpr (BITS == 4) bk[kk] = unpack(elem(kw, 2 * kk), elem(kw, 2 * kk + 1));
                    else bk[kk] = unpack(elem(kw, kk), 0u);
                }
            }
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb) {
                i32x4 r = mfma_i8(ak[rb][0], bk[0], zero);
#pragma unroll
                for (int kk = 1; kk < NKK; ++kk) r = mfma_i8(ak[rb][kk], bk[kk], r);
                if constexpr (KT) {
                    const auto kmw = whole(cur.km[sb]);
                    sc[rb][sb] = __uint_as_float(elem(kmw, 0)) *
                                 (combine(r) * kinv_l[rb] - (__uint_as_float(elem(kmw, 1)) - ZOFF) * kqs_l[rb]);
                } else {
                    sc[rb][sb] = combine(r) * kinv_l[rb] - kbias_l[rb];
                }
                if constexpr (SP) {  // rows of absent heads read a valid head's term, unused
                    const int head = min(4 * rb + (lane >> 4), GQ - 1);
                    sc[rb][sb] += (float)kc[head * GT + tig * TM + 16 * sb + (lane & 15)] * kc_inv;
                }
            }
        }
        uint8_t* avb = av_lds + buf * AV_BYTES;
        float vinv[RBK][NVG];
        float sp_val[SP ? RBK : 1][SP ? NVG : 1][SP ? NSB : 1];  // SP: value outlier terms and places
        int sp_idx[SP ? RBK : 1][SP ? NVG : 1][SP ? NSB : 1];
        const int tok = lane & 15, row = 4 * (lane >> 4);
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb) {
            float mt = sc[rb][0];
#pragma unroll
            for (int sb = 1; sb < NSB; ++sb) mt = fmaxf(mt, sc[rb][sb]);
            mt = group_max<16>(mt);
            const float mn = fmaxf(m_l[rb], mt);
            const float f = fast_exp2(m_l[rb] - mn);  // 0 while m is -inf
            m_l[rb] = mn;
            l2[rb] *= f;
#pragma unroll
            for (int g = 0; g < NVG; ++g) z2[rb][g] *= f;
#pragma unroll
            for (int n = 0; n < NVM; ++n) acc2[rb][n] *= f;
            float p[NSB];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                p[sb] = fast_exp2(sc[rb][sb] - mn);
                l2[rb] += p[sb];
            }
#pragma unroll
            for (int g = 0; g < NVG; ++g) {
                float w[NSB], wmax = 0.0f;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const auto vmw = whole(cur.vm[sb]);
                    w[sb] = p[sb] * __uint_as_float(elem(vmw, 2 * g));
                    z2[rb][g] = fmaf(w[sb], __uint_as_float(elem(vmw, 2 * g + 1)) - ZOFF, z2[rb][g]);
                    wmax = fmaxf(wmax, w[sb]);
                    if constexpr (SP) {
                        // value outlier of (token 16 sb + l % 16, group g): p (x - (u - z) s) onto
                        // its channel, added after the weights are read back; rows of absent heads
                        // add nothing
                        const int head = 4 * rb + (lane >> 4);
                        const uint32_t e = (cur.voi[sb] >> (NVG == 1 ? voi_shift : 16 * g)) & 0xFFFFu;
                        const float dv = __uint_as_float(elem(whole(cur.vov[sb]), g)) -
                                         ((float)(e >> 8) - __uint_as_float(elem(vmw, 2 * g + 1))) *
                                             __uint_as_float(elem(vmw, 2 * g));
                        sp_val[rb][g][sb] = head < GQ ? p[sb] * dv : 0.0f;
                        sp_idx[rb][g][sb] = min(head, GQ - 1) * D + g * (D / NVG) + (int)(e & 0xFFu);
                    }
                }
                const FixScale fs = fix_scale(group_max<16>(wmax));
                vinv[rb][g] = fs.inv;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const uint32_t d = digits256((int)rintf(w[sb] * fs.mul));
                    uint8_t* dst = avb + ((g * RBK + rb) * 16 + row) * 64 + 16 * sb + tok;
                    dst[0] = (uint8_t)d;
                    dst[64] = (uint8_t)(d >> 8);
                    dst[128] = (uint8_t)(d >> 16);
                }
            }
        }
        wave_lds_sync();
        i32x4 av[NVG][RBK];
#pragma unroll
        for (int g = 0; g < NVG; ++g)
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb)
                av[g][rb] = *reinterpret_cast<const i32x4*>(avb + ((g * RBK + rb) * 16 + (lane & 15)) * 64 + (lane >> 4) * 16);
        float vc_inv = 0.0f;
        if constexpr (SP) {
            // after the weights' reads (LDS keeps a wave's operations in order): the atomics'
            // latency overlaps the value products, and the read-back below comes after them.
            // Fixed point as for the keys: each term below 2^24 units of the tile's
            // largest, at most TM terms per (head, channel).
            float vmx = 0.0f;
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
                for (int g = 0; g < NVG; ++g)
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) vmx = fmaxf(vmx, fabsf(sp_val[rb][g][sb]));
            const FixScale fs = fix_scale(group_max<64>(vmx));
            const float vmul = fs.mul * 64.0f;
            vc_inv = fs.inv * (1.0f / 64.0f);
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
                for (int g = 0; g < NVG; ++g)
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb)
                        atomicAdd(&vc[sp_idx[rb][g][sb]], (int)rintf(sp_val[rb][g][sb] * vmul));
        }
#pragma unroll
        for (int m = 0; m < NVB; ++m) {
            u32x4 w[VBB];
#pragma unroll
            for (int bb = 0; bb < VBB; ++bb) w[bb] = whole(cur.v[m][bb]);
            const int g = NVG == 1 ? 0 : m;  // two value groups: one per 64-channel block
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                i32x4 bv;
                if constexpr (BITS == 8) bv = i32x4{(int)w[0][i], (int)w[1][i], (int)w[2][i], (int)w[3][i]};
                else bv = unpack(w[0][i], w[VBB - 1][i]);
#pragma unroll
                for (int rb = 0; rb < RBK; ++rb) {
                    const i32x4 r = mfma_i8(av[g][rb], bv, zero);
                    acc2[rb][4 * m + i] = fmaf(combine(r), vinv[rb][g], acc2[rb][4 * m + i]);
                }
            }
        }
        if constexpr (SP) {
            // this tile's value outlier terms of the lane's (head, channel) accumulators,
            // then cleared for the next tile (rows of absent heads read a valid head's)
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb) {
                const int head = min(4 * rb + (lane >> 4), GQ - 1);
#pragma unroll
                for (int n = 0; n < NVM; ++n) {
                    int* q = &vc[head * D + 64 * (n / 4) + 4 * (lane & 15) + (n % 4)];
                    acc2[rb][n] = fmaf((float)*q, vc_inv, acc2[rb][n]);
                    *q = 0;
                }
            }
        }
    }

    // The wave's key groups, through the tile ring (as in the VALU stream).
    __device__ __forceinline__ void run(int n_my_groups, const float (&qv)[GQ][KM]) {
        const int n_iter = n_my_groups / GB;
        int it = 0;
        if constexpr (KT) fold_kt(qv);
        auto step = [&](auto bc) __attribute__((always_inline)) {
            constexpr int B = decltype(bc)::value;
            constexpr int NB = B + NRM - 1;
            load(t[NB % NRM], it * GB + NB / TPG, NB % TPG, NB % TPG == 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!KT && B % TPG == 0) fold(t[B % NRM], qv);
            process(t[B % NRM], B & 1, B % TPG);
            __builtin_amdgcn_sched_barrier(0);
        };
        for (; it < n_iter; ++it) StaticFor<0, BODY>::run(step);
        if constexpr (GB > 1) {
            const int tail = (n_my_groups - n_iter * GB) * TPG;
            auto tail_step = [&](auto ic) __attribute__((always_inline)) {
                constexpr int I = decltype(ic)::value;
                if (tail > I) {
                    if constexpr (!KT && I % TPG == 0) fold(t[I], qv);
                    process(t[I], I & 1, I % TPG);
                }
            };
            StaticFor<0, NRM - TPG>::run(tail_step);
        }
    }

    // Merges the stream's state into the wave state of the VALU layout (running
    // max m, per-lane sums lpart and zpart, accumulators accv of channels
    // 32-lane-strided), and leaves the stream's accumulators, rescaled, in s_acc
    // ([GQ][D] floats of this wave) for the wave-state step to add.
    __device__ __forceinline__ void merge(float (&m)[GQ], float (&lpart)[GQ], float (&zpart)[GQ],
                                          float (&accv)[GQ][VCPL], float* s_acc) {
        const int hs = lane >> 4, j = lane & 15;
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const int rb = h / 4, hh = h % 4;
            const float m2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_l[rb]), 16 * hh));
            const float M = fmaxf(m[h], m2);
            const float f1 = m[h] == -INFINITY ? 0.0f : fast_exp2(m[h] - M);
            const float f2 = m2 == -INFINITY ? 0.0f : fast_exp2(m2 - M);
            m[h] = M;
            lpart[h] *= f1;
            zpart[h] *= f1;
#pragma unroll
            for (int c = 0; c < VCPL; ++c) accv[h][c] *= f1;
            const bool mine = hs == hh;
            lpart[h] += mine ? l2[rb] * f2 : 0.0f;
#pragma unroll
            for (int g = 0; g < NVG; ++g) {
                const float zs = group_sum<16>(z2[rb][g]);
                zpart[h] += (mine && j == g) ? zs * f2 : 0.0f;
            }
            if (mine) {
#pragma unroll
                for (int n = 0; n < NVM; ++n) s_acc[h * D + 64 * (n / 4) + 4 * j + (n % 4)] = acc2[rb][n] * f2;
            }
        }
        wave_lds_sync();
    }
};

// ---------------------------------------------------------------------------
// LDS carve-up (dynamic shared memory)
// ---------------------------------------------------------------------------
template <int D, int GQ, int TILE, int MFB = 0, int SPB = 0>
struct LdsPlan {
    // per wave: key digits [GQ][limb][D/2] paired bytes and an unread area of the
    // same size (written by the lanes of the pairs' upper channels), then two buffers of weight digits
    // [GQ][nvg][limb][TILE] bytes (alternating by tile), then the outlier
    // corrections of dense-and-sparse records (SPB bytes); with the matrix-core
    // stream, its operand rows (MFB bytes)
    __host__ __device__ static int valu_bytes(int nvg) {
        const int b = GQ * kLimbs * D + 2 * GQ * nvg * kLimbs * TILE;
        return (b + 15) & ~15;
    }
    __host__ __device__ static int wave_bytes(int nvg) {
        if (MFB > 0) return MFB + SPB;
        return valu_bytes(nvg) + SPB;
    }
    // per workgroup: wave states and the last-arrival flag
    __host__ __device__ static int wg_floats() { return kWaves * GQ * D + kWaves * GQ * 2 + 4; }
    __host__ __device__ static int bytes(int nvg) { return kWaves * wave_bytes(nvg) + 4 * wg_floats(); }
};

// ---------------------------------------------------------------------------
// the kernel: grid = (nsplit, BH)
// ---------------------------------------------------------------------------
// MF: the quantized stream runs on the matrix cores (MStream; TILE 64, TPG = G / 64,
// NVGT value groups per token); otherwise on the VALU with the CPL / TILE / TPG map.
// SP: dense-and-sparse records (one full-precision outlier per key channel group
// and per value group): the VALU stream adds each outlier's difference from its
// dequantized code to the scores and outputs.  SPW: caches with one value group
// per token, on a map with four key lanes and four tokens per slot.  KT: per-token
// keys (one scale and zero point per token over its D channels): the query is
// folded once per wave and every score takes its token's scale and zero point,
//   q . k'_t = s_t (sum_c q_c (u_tc - bias) - (z_t - bias) sum_c q_c).
template <int BITS, int D, int GQ, int CPL, int TILE, int TPG, bool MF = false, int NVGT = 1, bool SP = false,
          bool SPW = false, bool KT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(two_waves(MF, BITS, GQ, SP) ? 2 : 1)))
void decode_kernel(DecArgs a) {
    constexpr int LPT = D / CPL;           // key lanes per token
    constexpr int TPW = 64 / LPT;          // tokens per key wave-load
    constexpr int U = TILE / TPW;          // tokens per slot per tile
    // Code width of the VALU stream.  8-bit codes always take the matrix-core
    // stream (MF); their instantiations compile the VALU stream as 4-bit code
    // that never runs.
    constexpr int VB = BITS == 8 ? 4 : BITS;
    static_assert(BITS != 8 || MF, "8-bit codes run on the matrix-core stream only");
    constexpr int LW = CPL * VB / 32;      // packed key dwords per lane per token
    constexpr int KND = CPL / 8;           // key nibble dwords per lane per token
    constexpr int RB = D * VB / 8;         // key row bytes
    constexpr int TB = 32 / VB;            // tokens per value dword
    constexpr int VCPL = D / 32;           // value channels per lane
    constexpr int NVL = TILE / (2 * TB);   // value wave-loads per tile
    constexpr int VNE = TB / 8;            // nibble dwords per value code dword
    constexpr int KM = D / 64;             // channels per lane in the query fold
    constexpr int ZB = VB == 4 ? 8 : 0;    // code bias
    static_assert(LW >= 1 && LW * 32 == CPL * VB, "key lane chunk must be whole dwords");
    static_assert(U >= 1 && U * TPW == TILE, "tile must be whole key wave-loads");
    static_assert(NVL >= 1 && NVL * 2 * TB == TILE, "tile must be whole value wave-loads");
    static_assert(TPG == 1 || TPG == 2 || TPG == 4 || TPG == 8, "tiles per key group");
    static_assert(TILE % 32 == 0 && (U == 2 || U == 4 || U == 8), "digit runs of 2, 4 or 8 bytes");
    // A nibble dword of value codes pairs tokens t and t + PT in each byte (PT = 4
    // for 4-bit codes, 8 for 2-bit ones; pairs of a block of 2 PT tokens in order).
    // The U tokens of a key slot are UH such pairs, tokens tok0 + tok_off(u): the
    // slot's weight digits then go to LDS as bytes that already pair them, and
    // the value lanes read their digit dwords whole.
    constexpr int PT = VB == 4 ? 4 : 8;
    constexpr int UH = U / 2;
    static_assert(PT % UH == 0, "a slot's pairs lie in one block of 2 PT tokens");
    constexpr auto tok_off = [](int u) constexpr { return u % UH + PT * (u / UH); };

    extern __shared__ __align__(16) unsigned char dsm[];
    using MS = MStream<BITS, D, GQ, TPG, NVGT, SP, KT>;
    static_assert(!(KT && SP), "per-token keys take no outliers");
    // One value group per token (the host's choice) and as many key lanes per token
    // as tokens per slot: lane (slot, chunk) takes the value outlier of token
    // slot * U + chunk, the slot's four entries loading as one vector.
    constexpr bool SP_WIDE = SP && SPW;
    static_assert(!SPW || (SP && U == 4 && D / CPL == 4), "wide outlier map: four lanes and four tokens per slot");
    // outlier corrections: the key group's score terms [GQ][G], the tile's output terms [GQ][D]
    constexpr int SPB = SP ? 4 * (GQ * TILE * TPG + GQ * D) : 0;
    using LP = LdsPlan<D, GQ, TILE, MF ? MS::lds_bytes() : 0, SPB>;

    // grid = (nsplit, BH), or (BH, nsplit) with weighted splits (split_major: consecutive
    // workgroups are the same split of consecutive slices).  The host weights the splits
    // of the matrix-core stream run two workgroups per CU only; other instantiations
    // compile without the weighted plan.
    constexpr bool WSPLIT = MF && two_waves(MF, BITS, GQ, SP);
    const bool split_major = WSPLIT && a.split_major;
    const int split = split_major ? blockIdx.y : blockIdx.x;
    const int64_t bh = split_major ? blockIdx.x : blockIdx.y;
    const int b = (int)(bh / a.Hkv), kvh = (int)(bh % a.Hkv);
    // this slice's sinks, full-precision tokens and key groups
    int nS_s = a.nS, nfp_s = a.nfp, ng_s = a.ngroups;
    if (a.base_len != nullptr) {
        const SliceState st = slice_state((int64_t)a.base_len[b] + a.len_delta, a.S, a.R, a.Qf);
        nS_s = st.nS;
        nfp_s = st.nS + st.r;
        ng_s = st.Lq / a.G;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar, so that loop bounds and branches derived from it are
    // wave-uniform (scalar branches, no exec-mask loops)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nvg = a.nvg;

    uint8_t* kd = dsm + wave * LP::wave_bytes(nvg);            // key digits
    // SP: key outlier terms [GQ][G] (the matrix-core stream's own copy of this pointer is the same)
    // (both in fixed point: LDS integer atomics run far faster than float ones)
    int* kc = reinterpret_cast<int*>(kd + (MF ? MS::lds_bytes() : LP::valu_bytes(nvg)));
    int* vc = kc + GQ * TILE * TPG;                                  // SP: value outlier terms [GQ][D]
    float kc_inv = 0.0f;                                             // SP: 2^-k of the key group's terms
    if constexpr (SP)
        for (int i = lane; i < GQ * D; i += 64) vc[i] = 0;
    uint8_t* pd = kd + GQ * kLimbs * D;                         // weight digits (x2)
    float* wg = reinterpret_cast<float*>(dsm + kWaves * LP::wave_bytes(nvg));
    float* s_acc = wg;                                          // [kWaves][GQ][D]
    float* s_ml = s_acc + kWaves * GQ * D;                      // [kWaves][GQ][2]
    int* s_last = reinterpret_cast<int*>(s_ml + kWaves * GQ * 2);

    const int slot = lane / LPT, chunk = lane % LPT;
    const int sp0 = slot * UH;                                // the slot's first token pair
    const int tok0 = 2 * PT * (sp0 / PT) + sp0 % PT;         // its first token
    const int hb = lane >> 5;                  // value half: block parity
    const int c0v = (lane & 31) * VCPL;        // value channels of this lane
    const int gv = c0v / a.GV;                 // their value group
    // value scales: lane chunk < nvg of a key slot owns value group `chunk` of the
    // slot's tokens (nvg <= LPT); the other lanes load a valid duplicate
    const int gz = chunk & (nvg - 1);
    const bool owner = chunk < nvg;
    const int64_t qrow0 = (int64_t)b * a.Hkv * GQ + (int64_t)kvh * GQ;
    const char* const ksink = arg_ptr(a.ksink);
    const char* const vsink = arg_ptr(a.vsink);
    const char* const kres = arg_ptr(a.kres);
    const char* const vres = arg_ptr(a.vres);
    const char* const knew = arg_ptr(a.knew);
    const char* const vnew = arg_ptr(a.vnew);

    // Fused append: split 0 stores the newest token into its residual row (the
    // attention below reads it from the input, so no workgroup waits for this
    // store).  The row is loaded here, first of all loads, and stored after the
    // prologue, when it has long arrived.  esize * D bytes per row, a multiple
    // of 16; lanes [0, chunks) carry K, [chunks, 2 chunks) carry V.
    const bool copy_fresh = knew != nullptr && split == 0 && wave == kWaves - 1;
    uint4 fresh_word = make_uint4(0u, 0u, 0u, 0u);
    uint4* fresh_dst = nullptr;
    if (copy_fresh) {
        const int es = a.dtype == DT_F32 ? 4 : 2;
        const int chunks = D * es / 16;
        const int64_t dst_row = bh * a.R + (nfp_s - 1 - nS_s);
        if (lane < 2 * chunks) {
            const bool is_v = lane >= chunks;
            const int c = is_v ? lane - chunks : lane;
            fresh_word = reinterpret_cast<const uint4*>((is_v ? vnew : knew) + bh * D * es)[c];
            fresh_dst = reinterpret_cast<uint4*>(const_cast<char*>(is_v ? vres : kres) + dst_row * D * es) + c;
        }
    }

    float m[GQ], lpart[GQ], zpart[GQ], accv[GQ][VCPL];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        m[h] = -INFINITY;
        lpart[h] = 0.0f;
        zpart[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < VCPL; ++c) accv[h][c] = 0.0f;
    }

    // Rescales the state when the wave-uniform running max grows.
    auto update_max = [&](const float (&mt)[GQ]) __attribute__((always_inline)) {
        bool grow = false;
        float mnew[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            mnew[h] = fmaxf(m[h], mt[h]);
            grow |= mnew[h] > m[h];
        }
        if (wave_any(grow)) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float f = fast_exp2(m[h] - mnew[h]);
                m[h] = mnew[h];
                lpart[h] *= f;
                zpart[h] *= f;
#pragma unroll
                for (int c = 0; c < VCPL; ++c) accv[h][c] *= f;
            }
        }
    };

    // ---------------- quantized key groups of this split ----------------
    // The loop over the wave's key groups (TILE * TPG tokens each) is unrolled over
    // BODY tiles (whole groups) and is free of branches: the query fold of a group sits at a
    // fixed position in the body, and every tile rescales the softmax state and
    // turns its value dot products into fp32.  (A branch in the loop body makes the
    // compiler copy the tile buffers at the back edge, which waits for the loads in
    // flight and serialises the memory stream.)
    // Ring of NR tile buffers: NR - 1 tiles in flight while one is processed.
    constexpr int NR = two_waves(false, BITS, GQ, SP) ? 2 : 4;
    constexpr int BODY = TPG > NR ? TPG : NR;  // tiles per loop iteration (2, 4 or 8)
    constexpr int GB = BODY / TPG;             // key groups per loop iteration
    // splits 0 .. s1 - 1 take gps key groups each, the others gps2 (fewer where the
    // host weights the splits, see the split plan)
    const bool first = !WSPLIT || split < a.s1;
    const int g_begin = first ? split * a.gps : a.s1 * a.gps + (split - a.s1) * a.gps2;
    const int g_end = min(g_begin + (first ? a.gps : a.gps2), ng_s);
    const int n_my_groups = g_begin + wave < g_end ? (g_end - g_begin - wave + kWaves - 1) / kWaves : 0;

    {
        // the records of this slice: its own contiguous stream, or pages of the pool
        __amdgpu_buffer_rsrc_t rs;
        GroupAddr ga;
        ga.g0 = g_begin + wave;
        ga.rec_bytes = (uint32_t)a.rec_bytes;
        ga.gmax = a.table == nullptr ? max((int)a.ng_cap - 1, 0) : 0x7FFFFFFF;
        if (a.table == nullptr) {
            rs = make_rsrc(a.rec + (size_t)bh * (size_t)a.ng_cap * (size_t)a.rec_bytes,
                           (uint32_t)(a.ng_cap * a.rec_bytes));
            ga.lp = 31;
            ga.mask = 0x7FFFFFFFu;
            ga.p_first = 0;
            ga.page_off = 0u;
        } else {
            rs = make_rsrc(a.rec, a.pool_bytes);
            ga.lp = a.lp;
            ga.mask = (1u << a.lp) - 1u;
            ga.p_first = g_begin >> a.lp;
            const int n_pages = ((max(g_end, g_begin + 1) - 1) >> a.lp) - ga.p_first + 1;  // <= 64
            // entries past a sequence's own pages may be stale: any page of the pool serves,
            // since those groups' words are never used
            int page = lane < n_pages ? a.table[(int64_t)b * a.max_pages + ga.p_first + lane] : 0;
            page = (uint32_t)page < (uint32_t)a.pool_pages ? page : 0;
            ga.page_off = (uint32_t)page * a.page_bytes + (uint32_t)kvh * ((uint32_t)a.rec_bytes << a.lp);
        }
        float qv[GQ][KM];  // folded query of this lane's KM channels (set in the prologue)
        MS ms;             // the matrix-core stream (MF only)
        if constexpr (MF) ms.init(a, rs, ga, n_my_groups, lane, kd);

        // One tile of the wave's stream.  Key token tok0 + tok_off(u) of the tile is
        // scored by the LPT lanes of `slot`; value block hb * NVL + vl (TB tokens)
        // of channels c0v.. is handled by this lane.  ks/kz (key scales and zero
        // points of this lane's KM fold channels) are loaded with a group's first tile.
        struct Tile {
            typename UVec<LW>::T k[U];
            typename UVec<VCPL>::T v[NVL];
            u32x2 vm[U];  // value scale, zero point (fp32 bits) of (token, group gz)
            u32x2 km[U];  // KT: key scale, zero point (fp32 bits) of each token
            typename UVec<KM>::T ks, kz;
            // SP only: the key outliers of the KM fold channels (values; dword of
            // (token | code << 8) u16 fields), the value outlier of (token, group gz)
            typename UVec<KM>::T kov;
            uint32_t koi;
            uint32_t vov[U], voi[U];
            // one value group per token (NVGT == 1, U == 4): the slot's four items at once
            u32x4 vov4;
            u32x2 voi4;
        };
        const int last_group = n_my_groups - 1;
        // per-lane byte offsets, the same for every tile
        const uint32_t k_off = (uint32_t)a.rec_kcodes + tok0 * RB + chunk * (LW * 4);
        const uint32_t v_off = (uint32_t)a.rec_vcodes + (hb * NVL * D + c0v) * 4;
        const uint32_t km_off = KM * lane * 4;
        uint32_t vm_off[U], kt_off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vm_off[u] = (uint32_t)a.rec_vmeta + ((tok0 + tok_off(u)) * nvg + gz) * 8;
            kt_off[u] = (tok0 + tok_off(u)) * 8;  // KT: the token's (scale, zero) at the record's start
        }
        // SP: outlier fields of this lane's fold channels and of its (token, group gz)
        // items; a u16 field is read with the dword that holds it
        const uint32_t kov_off = (uint32_t)a.rec_kov + KM * lane * 4;
        const uint32_t koi_off = (uint32_t)a.rec_koi + ((KM * lane * 2) & ~3);
        const int koi_shift = KM == 1 ? 16 * (lane & 1) : 0;
        uint32_t vov_off[U], voi_off[U];
        int voi_shift[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int item = (tok0 + tok_off(u)) * nvg + gz;
            vov_off[u] = (uint32_t)a.rec_vov + item * 4;
            voi_off[u] = (uint32_t)a.rec_voi + ((item * 2) & ~3);
            voi_shift[u] = 16 * (item & 1);
        }

        // Loads tile `tig` of the wave's key group j; groups past the last one
        // reload the last (the loop prefetches beyond its end).  A wave with no
        // group reads group 0 of its split's range, or past the records' end,
        // where buffer loads return zeros; those words are never used.
        auto load = [&](Tile& t, int j, int tig, bool kmeta) __attribute__((always_inline)) {
            const uint32_t grp = ga.at(min(j, max(last_group, 0)));
            const int t0 = tig * TILE;
#pragma unroll
            for (int u = 0; u < U; ++u) t.k[u] = bload<LW>(rs, k_off + tok_off(u) * RB, grp + t0 * RB);
#pragma unroll
            for (int vl = 0; vl < NVL; ++vl) t.v[vl] = bload<VCPL>(rs, v_off + vl * D * 4, grp + (t0 / TB) * D * 4);
#pragma unroll
            for (int u = 0; u < U; ++u) t.vm[u] = bload<2>(rs, vm_off[u], grp + t0 * nvg * 8);
            if constexpr (KT) {
#pragma unroll
                for (int u = 0; u < U; ++u) t.km[u] = bload<2>(rs, kt_off[u], grp + t0 * 8);
            }
            if (!KT && kmeta) {  // constant at every call site
                t.ks = bload<KM>(rs, km_off, grp);
                t.kz = bload<KM>(rs, km_off + D * 4, grp);
                if constexpr (SP) {
                    t.kov = bload<KM>(rs, kov_off, grp);
                    t.koi = bload<1>(rs, koi_off, grp);
                }
            }
            if constexpr (SP) {
                // item offsets within the group: t0 * nvg items before this tile (t0 even)
                if constexpr (SP_WIDE) {
                    // tokens tok0, tok0 + 1 and their partners tok0 + PT, tok0 + PT + 1 (tok0 even)
                    const u32x2 x0 = bload<2>(rs, vov_off[0], grp + t0 * 4);
                    const u32x2 x1 = bload<2>(rs, vov_off[UH], grp + t0 * 4);
                    t.vov4 = u32x4{x0.x, x0.y, x1.x, x1.y};
                    t.voi4 = u32x2{bload<1>(rs, voi_off[0], grp + t0 * 2), bload<1>(rs, voi_off[UH], grp + t0 * 2)};
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        t.vov[u] = bload<1>(rs, vov_off[u], grp + t0 * nvg * 4);
                        t.voi[u] = bload<1>(rs, voi_off[u], grp + t0 * nvg * 2);
                    }
                }
            }
        };

        uint32_t kl[GQ][kLimbs][KND];  // key digit dwords of this lane's channels
        float kinv[GQ], kbias[GQ];

        // This lane's key digit dwords, read back from the wave's paired digit bytes
        // (store_key_digits: limb li of head h at kd + (h * kLimbs + li) * D / 2, the
        // pairs of this lane's channels at chunk * CPL / 2).
        constexpr int KP = VB == 4 ? 4 : 8;  // channel distance of a code nibble pair
        static_assert(CPL % (2 * KP) == 0, "a lane's channels are whole pair blocks");
        auto load_kl = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < GQ; ++h)
#pragma unroll
                for (int li = 0; li < kLimbs; ++li) {
                    const uint8_t* base = kd + (h * kLimbs + li) * (D / 2) + chunk * (CPL / 2);
                    if constexpr (KND == 4) {
                        const u32x4 x = *reinterpret_cast<const u32x4*>(base);
                        kl[h][li][0] = x.x, kl[h][li][1] = x.y, kl[h][li][2] = x.z, kl[h][li][3] = x.w;
                    } else if constexpr (KND == 2) {
                        const u32x2 x = *reinterpret_cast<const u32x2*>(base);
                        kl[h][li][0] = x.x, kl[h][li][1] = x.y;
                    } else {
                        static_assert(KND == 1, "1, 2 or 4 digit dwords per limb");
                        kl[h][li][0] = lds32(base);
                    }
                }
        };
        // the folded query's digits of head h: n[j] of channel KM * lane + j
        auto store_kd = [&](int h, const int (&n)[KM]) __attribute__((always_inline)) {
            store_key_digits<KM, KP>(kd + h * kLimbs * (D / 2), kd + (GQ + h) * kLimbs * (D / 2), D / 2, lane, n);
        };

        // Folds the key scales of a group into the query, in fixed point: digit
        // dwords of rint(q_c s_c 2^k) for this lane's key channels, and the
        // zero-point term sum_c q_c s_c (z_c - bias).
        auto fold = [&](const Tile& cur) __attribute__((always_inline)) {
            float qt[GQ][KM], mx[GQ], bp[GQ];
            const auto ks = whole(cur.ks), kz = whole(cur.kz);
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                mx[h] = 0.0f;
                bp[h] = 0.0f;
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    qt[h][j] = qv[h][j] * __uint_as_float(elem(ks, j));
                    mx[h] = fmaxf(mx[h], fabsf(qt[h][j]));
                    bp[h] = fmaf(qt[h][j], __uint_as_float(elem(kz, j)) - (float)ZB, bp[h]);
                }
            }
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const FixScale fs = fix_scale(group_max<64>(mx[h]));
                kinv[h] = fs.inv;
                kbias[h] = group_sum<64>(bp[h]);
                int n[KM];
#pragma unroll
                for (int j = 0; j < KM; ++j) n[j] = (int)rintf(qt[h][j] * fs.mul);
                store_kd(h, n);
            }
            if constexpr (SP) {
                // key outliers: q_c (x_c - (u_c - z_c) s_c) onto the score of token t_c
                // of the group, through a per-wave table (zeroed, then added to; LDS
                // keeps one wave's operations in order), in fixed point: each term below
                // 2^23 units of the group's largest, at most D terms per token
                constexpr int GT = TILE * TPG;
                const auto kov = whole(cur.kov);
                float kt[KM][GQ], kmx = 0.0f;
                int tk[KM];
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    const uint32_t e = (cur.koi >> (KM == 1 ? koi_shift : 16 * j)) & 0xFFFFu;
                    const float delta = __uint_as_float(elem(kov, j)) -
                                        ((float)(e >> 8) - __uint_as_float(elem(kz, j))) * __uint_as_float(elem(ks, j));
                    tk[j] = (int)(e & 0xFFu);
#pragma unroll
                    for (int h = 0; h < GQ; ++h) {
                        kt[j][h] = qv[h][j] * delta;
                        kmx = fmaxf(kmx, fabsf(kt[j][h]));
                    }
                }
                const FixScale fs = fix_scale(group_max<64>(kmx));
                const float kmul = fs.mul * 32.0f;
                kc_inv = fs.inv * (1.0f / 32.0f);
#pragma unroll
                for (int h = 0; h < GQ; ++h)
#pragma unroll
                    for (int i = 0; i < (GT + 63) / 64; ++i) kc[h * GT + ((i * 64 + lane) & (GT - 1))] = 0;
#pragma unroll
                for (int j = 0; j < KM; ++j)
#pragma unroll
                    for (int h = 0; h < GQ; ++h) atomicAdd(&kc[h * GT + tk[j]], (int)rintf(kt[j][h] * kmul));
            }
            wave_lds_sync();
            load_kl();
        };

        // Per-token keys: the query's digits (no key scale folded in), once per wave,
        // with 2^-k and the image's channel sum kqs = sum_c n_c 2^-k.
        float kqs[GQ];
        auto fold_kt = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float mx = 0.0f;
#pragma unroll
                for (int j = 0; j < KM; ++j) mx = fmaxf(mx, fabsf(qv[h][j]));
                const FixScale fs = fix_scale(group_max<64>(mx));
                kinv[h] = fs.inv;
                kbias[h] = 0.0f;
                float nsum = 0.0f;
                int n[KM];
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    n[j] = (int)rintf(qv[h][j] * fs.mul);
                    nsum += (float)n[j];
                }
                store_kd(h, n);
                kqs[h] = group_sum<64>(nsum) * fs.inv;
            }
            wave_lds_sync();
            load_kl();
        };

        // One tile: scores, softmax update, weight digits through LDS (buffer pb of
        // two, alternating by tile), value dot products folded into fp32.
        auto process = [&](const Tile& cur, uint8_t* pb, int tig) __attribute__((always_inline)) {
            // ---- key scores of this slot's U tokens ----
            float sc[GQ][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t cw[KND];
                const auto kw = whole(cur.k[u]);
#pragma unroll
                for (int d = 0; d < LW; ++d) {
                    if constexpr (VB == 4) {
                        cw[d] = elem(kw, d);  // fields are already code - 8
                    } else {
                        cw[2 * d] = elem(kw, d) & 0x33333333u;
                        cw[2 * d + 1] = (elem(kw, d) >> 2) & 0x33333333u;
                    }
                }
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    int acc = dot8_0(kl[h][kLimbs - 1][0], cw[0]);
#pragma unroll
                    for (int nd = 1; nd < KND; ++nd) acc = dot8(kl[h][kLimbs - 1][nd], cw[nd], acc);
#pragma unroll
                    for (int li = kLimbs - 2; li >= 0; --li) {
                        acc <<= 4;
#pragma unroll
                        for (int nd = 0; nd < KND; ++nd) acc = dot8(kl[h][li][nd], cw[nd], acc);
                    }
                    sc[h][u] = (float)acc;
                }
            }
            // ---- online softmax: wave-uniform running max, rescaled every tile ----
            float vinv[GQ];
            float vcinv[SP ? GQ : 1];  // SP: 2^-k of the value outlier terms of head h
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float mt = -INFINITY;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if constexpr (KT) {
                        const u32x2 km = whole(cur.km[u]);
                        sc[h][u] = __uint_as_float(km.x) *
                                   (group_sum<LPT>(sc[h][u]) * kinv[h] - (__uint_as_float(km.y) - (float)ZB) * kqs[h]);
                    } else {
                        sc[h][u] = group_sum<LPT>(sc[h][u]) * kinv[h] - kbias[h];
                    }
                    if constexpr (SP) sc[h][u] += (float)kc[h * TILE * TPG + tig * TILE + tok0 + tok_off(u)] * kc_inv;
                    mt = fmaxf(mt, sc[h][u]);
                }
                mt = slots_max<LPT>(mt);
                const float mn = fmaxf(m[h], mt);
                const float f = fast_exp2(m[h] - mn);  // 0 while m is -inf
                m[h] = mn;
                lpart[h] *= f;
                zpart[h] *= f;
#pragma unroll
                for (int c = 0; c < VCPL; ++c) accv[h][c] *= f;

                // ---- weights p_t s_t -> fixed-point digits in LDS ----
                float pt[U], mx = 0.0f;
                float pw[U];  // SP_WIDE: the tokens' softmax weights
                float vt[SP ? U : 1];  // SP: value outlier terms p (x - (u - z) s) and their channels
                int vi[SP ? U : 1];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float p = fast_exp2(sc[h][u] - mn);
                    const u32x2 vm = whole(cur.vm[u]);
                    pt[u] = p * __uint_as_float(vm.x);
                    // each (token, value group) counted by one lane, each token once
                    zpart[h] = fmaf(owner ? pt[u] : 0.0f, __uint_as_float(vm.y) - (float)ZB, zpart[h]);
                    lpart[h] += chunk == 0 ? p : 0.0f;
                    mx = fmaxf(mx, pt[u]);
                    if constexpr (SP && !SP_WIDE) {
                        // value outlier of (token, group gz): p (x - (u - z) s) onto its channel
                        const uint32_t e = (cur.voi[u] >> voi_shift[u]) & 0xFFFFu;
                        const float dv = __uint_as_float(cur.vov[u]) -
                                         ((float)(e >> 8) - __uint_as_float(vm.y)) * __uint_as_float(vm.x);
                        vt[u] = owner ? p * dv : 0.0f;
                        vi[u] = h * D + gz * a.GV + (int)(e & 0xFFu);
                    }
                    if constexpr (SP_WIDE) pw[u] = p;
                }
                if constexpr (SP_WIDE) {
                    // this lane's token of the slot (u = chunk): its value outlier's term
                    // (element-wise selects, no branches)
                    float pc = pw[0];
                    u32x2 vmc = whole(cur.vm[0]);
                    uint32_t xv = cur.vov4.x;
#pragma unroll
                    for (int u = 1; u < 4; ++u) {
                        const bool sel = chunk == u;
                        const u32x2 vmu = whole(cur.vm[u]);
                        pc = sel ? pw[u] : pc;
                        vmc.x = sel ? vmu.x : vmc.x;
                        vmc.y = sel ? vmu.y : vmc.y;
                        xv = sel ? elem(cur.vov4, u) : xv;
                    }
                    const uint32_t e = ((chunk < 2 ? cur.voi4.x : cur.voi4.y) >> (16 * (chunk & 1))) & 0xFFFFu;
                    const float dv = __uint_as_float(xv) - ((float)(e >> 8) - __uint_as_float(vmc.y)) * __uint_as_float(vmc.x);
                    vt[0] = pc * dv;
                    vi[0] = h * D + (int)(e & 0xFFu);
                }
                if constexpr (SP) {
                    // the tile's value outlier terms of head h into the table in fixed point:
                    // each below 2^24 units of the largest, at most TILE terms per channel
                    constexpr int NT = SP_WIDE ? 1 : U;
                    float vmx = 0.0f;
#pragma unroll
                    for (int u = 0; u < NT; ++u) vmx = fmaxf(vmx, fabsf(vt[u]));
                    const FixScale vfs = fix_scale(group_max<64>(vmx));
                    const float vmul = vfs.mul * 64.0f;
                    vcinv[h] = vfs.inv * (1.0f / 64.0f);
#pragma unroll
                    for (int u = 0; u < NT; ++u) atomicAdd(&vc[vi[u]], (int)rintf(vt[u] * vmul));
                }
                const FixScale fs = fix_scale(group_max<64>(mx));
                vinv[h] = fs.inv;
                int n[U];
#pragma unroll
                for (int u = 0; u < U; ++u) n[u] = (int)rintf(pt[u] * fs.mul);
                // the slot's pair bytes (every lane of a (slot, value group) writes the same bytes)
                store_pair_digits<U>(pb + ((h * nvg + gz) * kLimbs) * TILE + sp0, TILE, n);
            }
            wave_lds_sync();

            // ---- values: integer dot products along tokens, digits by Horner ----
            uint32_t vw[NVL][VCPL][VNE];
#pragma unroll
            for (int vl = 0; vl < NVL; ++vl) {
                const auto vv = whole(cur.v[vl]);
#pragma unroll
                for (int c = 0; c < VCPL; ++c) {
                    if constexpr (VB == 4) {
                        vw[vl][c][0] = elem(vv, c);  // fields are already code - 8
                    } else {
                        vw[vl][c][0] = elem(vv, c) & 0x33333333u;
                        vw[vl][c][VNE - 1] = (elem(vv, c) >> 2) & 0x33333333u;
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const uint8_t* pbase = pb + ((h * nvg + gv) * kLimbs) * TILE + hb * (TILE / 4);
                int acc[VCPL];
#pragma unroll
                for (int c = 0; c < VCPL; ++c) acc[c] = 0;
#pragma unroll
                for (int li = kLimbs - 1; li >= 0; --li) {
                    // pair bytes of this half's TILE / 2 tokens: digit dwords that line up
                    // with its value code nibble dwords
                    uint32_t w[TILE / 16];
                    if constexpr (TILE / 16 == 4) {
                        const u32x4 x = *reinterpret_cast<const u32x4*>(pbase + li * TILE);
                        w[0] = x.x, w[1] = x.y, w[2] = x.z, w[3] = x.w;
                    } else {
                        static_assert(TILE / 16 == 2, "32- or 64-token tiles");
                        const u32x2 x = *reinterpret_cast<const u32x2*>(pbase + li * TILE);
                        w[0] = x.x, w[1] = x.y;
                    }
#pragma unroll
                    for (int c = 0; c < VCPL; ++c) acc[c] <<= 4;
#pragma unroll
                    for (int vl = 0; vl < NVL; ++vl) {
                        uint32_t dl[VNE];
#pragma unroll
                        for (int e = 0; e < VNE; ++e) dl[e] = w[vl * VNE + e];
#pragma unroll
                        for (int c = 0; c < VCPL; ++c)
#pragma unroll
                            for (int e = 0; e < VNE; ++e) {
                                // the first product of a channel starts its sum
                                if (li == kLimbs - 1 && vl == 0 && e == 0) acc[c] = dot8_0(dl[e], vw[vl][c][e]);
                                else acc[c] = dot8(dl[e], vw[vl][c][e], acc[c]);
                            }
                    }
                }
#pragma unroll
                for (int c = 0; c < VCPL; ++c) accv[h][c] = fmaf((float)acc[c], vinv[h], accv[h][c]);
                if constexpr (SP) {
                    // this tile's value outlier terms of the lane's channels (taken by one
                    // lane of the two that hold them), then cleared for the next tile
#pragma unroll
                    for (int c = 0; c < VCPL; ++c) {
                        const float x = (float)vc[h * D + c0v + c] * vcinv[h];
                        accv[h][c] += hb == 0 ? x : 0.0f;
                        vc[h * D + c0v + c] = 0;
                    }
                }
            }
        };

        // The tile ring.  Step B of the body processes body tile B (group
        // B / TPG of the iteration, tile B % TPG) from buffer B % NR and
        // prefetches body tile B + NR - 1 into buffer (B + NR - 1) % NR.  The
        // scheduling barriers keep each buffer's new loads below the last use of
        // its old contents and issue the prefetch before the wait for the
        // current tile.
        uint8_t* pd0 = pd;
        uint8_t* pd1 = pd + GQ * nvg * kLimbs * TILE;
        Tile tr[NR];

        // ---------------- prologue: full-precision tokens (sinks, residual) ---------
        // The sinks and residual tokens of the split are scored while the first
        // quantized tiles are in flight, with a lane map of their own (CPLF channels
        // per lane, few registers).  Load order: query words, the first iteration's
        // key and value rows, then the tile prefetch; everything up to the first
        // iteration's arithmetic is straight-line code for one storage dtype, so
        // each wait is for its own loads only, not for the prefetch behind them.
        // Rows past the split's end reload its first row (row 0 when the slice has no
        // full-precision token, which may never have been written); their scores are
        // -inf and their value terms are skipped by selects.
        const int f0 = (int)((int64_t)split * nfp_s / a.nsplit);
        const int f1 = (int)((int64_t)(split + 1) * nfp_s / a.nsplit);
        constexpr int CPLF = 16;          // key channels per lane
        constexpr int LPTF = D / CPLF;    // lanes per token
        constexpr int TPWF = 64 / LPTF;   // tokens per wave step
        const int slotf = lane / LPTF, chunkf = lane % LPTF;
        // Byte address of element e0 of full-precision token j's key (or value) row:
        // sinks first, then the residual; with a fused append the newest token
        // comes from the caller's input.  Chosen by integer selects on finished
        // addresses (selects between the argument pointers would make the compiler
        // copy the kernel arguments to scratch memory).
        auto row_addr = [&](int j, int64_t e0, int es, bool key) -> const char* {
            typedef __attribute__((address_space(1))) const char gchar;
            const int64_t erow = (int64_t)D * es;
            const uint64_t a_sink = reinterpret_cast<uint64_t>(key ? ksink : vsink) + (bh * a.S + j) * erow;
            const uint64_t a_res = reinterpret_cast<uint64_t>(key ? kres : vres) + (bh * a.R + (j - nS_s)) * erow;
            const uint64_t a_new = reinterpret_cast<uint64_t>(key ? knew : vnew) + bh * erow;
            const bool fresh = knew != nullptr && j == nfp_s - 1;
            const uint64_t x = (fresh ? a_new : j < nS_s ? a_sink : a_res) + e0 * es;
            return (const char*)reinterpret_cast<gchar*>(x);
        };
        auto prologue = [&](auto dtc) __attribute__((always_inline)) {
            constexpr int DT = decltype(dtc)::value;
            constexpr int ES = DT == DT_F32 ? 4 : 2;  // bytes per element
            constexpr int KW = CPLF * ES / 4;         // key dwords per lane and token
            constexpr int VW = VCPL * ES / 4;         // value dwords per lane and token
            uint32_t qv_w[GQ][KM], qf_w[GQ][CPLF];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const char* qv_p = reinterpret_cast<const char*>(a.q) + ((qrow0 + h) * D + KM * lane) * ES;
                if constexpr (KM * ES >= 4) load_dwords(qv_p, qv_w[h], KM * ES / 4);
                else qv_w[h][0] = *reinterpret_cast<const uint16_t*>(qv_p);  // one 16-bit element
                load_dwords(reinterpret_cast<const char*>(a.q) + ((qrow0 + h) * D + chunkf * CPLF) * ES, qf_w[h], KW);
            }
            // Two wave steps (2 x TPWF tokens) per iteration: the rows of both are
            // loaded, still packed, before either is scored.
            uint32_t kw[2][KW];
            uint32_t vw[2][TPWF / 2][VW];  // value rows: half hb takes slots hb, hb + 2, ...
            auto load_iter = [&](int j00) __attribute__((always_inline)) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int j0 = j00 + st * kWaves * TPWF;
                    const int j = j0 + slotf;
                    load_dwords(row_addr(j < f1 ? j : f0, chunkf * CPLF, ES, true), kw[st], KW);
#pragma unroll
                    for (int k = 0; k < TPWF / 2; ++k) {
                        const int jt = j0 + 2 * k + hb;
                        load_dwords(row_addr(jt < f1 ? jt : f0, c0v, ES, false), vw[st][k], VW);
                    }
                }
            };
            const int jfirst = f0 + wave * TPWF;
            load_iter(jfirst);
            auto load_first = [&](auto ic) __attribute__((always_inline)) {
                constexpr int I = decltype(ic)::value;
                load(tr[I], I / TPG, I % TPG, I % TPG == 0);
                // tiles issue in ring order: the loop's waits count on it
                __builtin_amdgcn_sched_barrier(0);
            };
            if constexpr (MF) ms.start();
            else StaticFor<0, NR - 1>::run(load_first);
            __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
            float qf[GQ][CPLF];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
#pragma unroll
                for (int j = 0; j < KM; ++j) qv[h][j] = packed_f32<DT>(qv_w[h], j) * a.qscale;
#pragma unroll
                for (int c = 0; c < CPLF; ++c) qf[h][c] = packed_f32<DT>(qf_w[h], c) * a.qscale;
            }
            auto score_iter = [&](int j00) __attribute__((always_inline)) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int j0 = j00 + st * kWaves * TPWF;
                    const bool valid = j0 + slotf < f1;
                    float sc[GQ];
#pragma unroll
                    for (int h = 0; h < GQ; ++h) {
                        float t = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPLF; ++c) t = fmaf(qf[h][c], packed_f32<DT>(kw[st], c), t);
                        t = group_sum<LPTF>(t);
                        sc[h] = valid ? t : -INFINITY;
                    }
                    float mt[GQ];
#pragma unroll
                    for (int h = 0; h < GQ; ++h) mt[h] = slots_max<LPTF>(sc[h]);
                    update_max(mt);
                    float pv[GQ];
#pragma unroll
                    for (int h = 0; h < GQ; ++h) {
                        pv[h] = valid ? fast_exp2(sc[h] - m[h]) : 0.0f;
                        if (chunkf == 0) lpart[h] += pv[h];
                    }
#pragma unroll
                    for (int k = 0; k < TPWF / 2; ++k) {
                        const int sl = 2 * k + hb;
                        // a row past the split's end holds a reloaded row that may never have
                        // been written (no full-precision token at all): it is skipped by a
                        // select, since a zero weight times non-finite bits is not zero
                        const bool vsl = j0 + sl < f1;
#pragma unroll
                        for (int h = 0; h < GQ; ++h) {
                            const float psl = __shfl(pv[h], sl * LPTF);
#pragma unroll
                            for (int c = 0; c < VCPL; ++c) {
                                const float nv = fmaf(psl, packed_f32<DT>(vw[st][k], c), accv[h][c]);
                                accv[h][c] = vsl ? nv : accv[h][c];
                            }
                        }
                    }
                }
            };
            score_iter(jfirst);  // a no-op when the split has no full-precision token here
            for (int j00 = jfirst + 2 * kWaves * TPWF; j00 < f1; j00 += 2 * kWaves * TPWF) {
                load_iter(j00);
                score_iter(j00);
            }
        };
        if (a.dtype == DT_BF16) prologue(std::integral_constant<int, DT_BF16>());
        else if (a.dtype == DT_F16) prologue(std::integral_constant<int, DT_F16>());
        else prologue(std::integral_constant<int, DT_F32>());
        if (fresh_dst != nullptr) *fresh_dst = fresh_word;

        // ---------------- the quantized stream ----------------
        if constexpr (MF) {
            if (n_my_groups > 0) ms.run(n_my_groups, qv);
            ms.merge(m, lpart, zpart, accv, s_acc + wave * GQ * D);
        } else if (n_my_groups > 0) {
            const int n_iter = n_my_groups / GB;
            int it = 0;
            if constexpr (KT) fold_kt();
            auto step = [&](auto bc) __attribute__((always_inline)) {
                constexpr int B = decltype(bc)::value;
                constexpr int NB = B + NR - 1;  // body tile to prefetch (may be in the next iteration)
                load(tr[NB % NR], it * GB + NB / TPG, NB % TPG, NB % TPG == 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!KT && B % TPG == 0) fold(tr[B % NR]);
                process(tr[B % NR], (B & 1) ? pd1 : pd0, B % TPG);
                __builtin_amdgcn_sched_barrier(0);
            };
            // Issue priority by progress: the wave's iterations run in quarters at
            // priority 3, 2, 1 and 0.  Of two workgroups on a CU, the SIMDs otherwise
            // favour the older one's waves throughout, so the younger falls behind and
            // its slot ends last; now the one with less of its stream done wins, and
            // the two run closer to level.
            // (One loop: the priority changes by scalar branches at the quarter
            // boundaries, outside the unrolled body.)
            const int q1 = n_iter / 4, q2 = n_iter / 2, q3 = 3 * n_iter / 4;
            __builtin_amdgcn_s_setprio(3);
            for (; it < n_iter; ++it) {
                if (it == q1) __builtin_amdgcn_s_setprio(2);
                if (it == q2) __builtin_amdgcn_s_setprio(1);
                if (it == q3) __builtin_amdgcn_s_setprio(0);
                StaticFor<0, BODY>::run(step);
            }
            // Groups after the last whole iteration: fewer than GB, so at most
            // NR - TPG tiles, already in the first NR - 1 buffers.
            if constexpr (GB > 1) {
                const int tail = (n_my_groups - n_iter * GB) * TPG;
                auto tail_step = [&](auto ic) __attribute__((always_inline)) {
                    constexpr int I = decltype(ic)::value;
                    if (tail > I) {
                        if constexpr (!KT && I % TPG == 0) fold(tr[I]);
                        process(tr[I], (I & 1) ? pd1 : pd0, I % TPG);
                    }
                };
                StaticFor<0, NR - TPG>::run(tail_step);
            }
        }
    }

    // ---------------- wave state -> LDS ----------------
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        const float L = group_sum<64>(lpart[h]);
        // zpart of lane l belongs to value group l % nvg; Zv is the total of this
        // lane's channel group gv (nvg is a power of two, wave-uniform)
        float Zv = 0.0f;
        for (int g = 0; g < nvg; ++g) {
            const float Zg = group_sum<64>((lane & (nvg - 1)) == g ? zpart[h] : 0.0f);
            Zv = gv == g ? Zg : Zv;
        }
#pragma unroll
        for (int c = 0; c < VCPL; ++c) {
            const float tot = accv[h][c] + __shfl_xor(accv[h][c], 32) - Zv;
            float* dst = &s_acc[(wave * GQ + h) * D + c0v + c];
            if (lane < 32) *dst = MF ? *dst + tot : tot;  // MF: the stream's part is already there
        }
        if (lane == 0) {
            s_ml[(wave * GQ + h) * 2] = m[h];
            s_ml[(wave * GQ + h) * 2 + 1] = L;
        }
    }
    __syncthreads();

    // ---------------- merge the waves of this workgroup ----------------
    const bool single = a.nsplit == 1;
    for (int e = tid; e < GQ * D; e += kThreads) {
        const int h = e / D, c = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[(w * GQ + h) * 2]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = s_ml[(w * GQ + h) * 2];
            const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
            L = fmaf(s_ml[(w * GQ + h) * 2 + 1], f, L);
            A = fmaf(s_acc[(w * GQ + h) * D + c], f, A);
        }
        if (single) {
            a.out[(qrow0 + h) * D + c] = A / L;
            if (c == 0 && a.lse) a.lse[qrow0 + h] = (M + __log2f(L)) * 0.69314718055994530942f;
        } else {
            const int64_t pidx = (bh * a.nsplit_cap + split) * GQ + h;
            publish(&a.part_acc[pidx * D + c], A);
            if (c == 0) {
                publish(&a.part_ml[pidx * 2], M);
                publish(&a.part_ml[pidx * 2 + 1], L);
            }
        }
    }
    if (single) return;

    // Split combine by last arrival, in one level or two.  With a.cgs < nsplit the
    // splits form groups of a.cgs consecutive splits: the last arrival of a group
    // merges the group's partials into a group partial, and the last group merger
    // of the slice merges the group partials into the output.  The merges of the
    // early groups overlap the streams still running, and no workgroup reads more
    // than max(a.cgs, groups) partials (one workgroup reading all of a long slice's
    // partials through device-scope loads would otherwise set the kernel's end).
    // With a.cgs >= nsplit the slice's last arrival merges every split.
    //
    // Ordering.  Every value exchanged between workgroups (partials, counters) is
    // written and read with device-scope accesses, which the hardware performs at
    // the device's coherence point rather than in one XCD's L2, so no L2
    // write-back or invalidate is needed.  A publishing workgroup's stores must be
    // complete before its arrival is counted: every wave waits until all its
    // memory operations are acknowledged (s_waitcnt 0; the signal fences around it
    // keep the compiler from moving memory accesses across the wait), and the
    // workgroup barrier puts every wave's wait before the one thread's atomic add
    // on the counter.  The merger issues its loads only after that add has returned
    // the count that makes it last: the branch on the count (through LDS and a
    // barrier) precedes every load of the merge.
    const int ng1 = (a.nsplit + a.cgs - 1) / a.cgs;  // groups of the first level
    const int grp = split / a.cgs;
    const float* pml = a.part_ml + (bh * a.nsplit_cap + (int64_t)grp * a.cgs) * GQ * 2;
    const float* pacc = a.part_acc + (bh * a.nsplit_cap + (int64_t)grp * a.cgs) * GQ * D;
    int ns = min(a.cgs, a.nsplit - grp * a.cgs);  // partials the next merge takes
    // slice counter at [bh]; with two levels, group counters at [BH + bh * cgroups_cap + grp]
    const int64_t n_slices = split_major ? gridDim.x : gridDim.y;
    unsigned* ctr = ng1 > 1 ? a.counters + n_slices + bh * a.cgroups_cap + grp : a.counters + bh;
    bool final = ng1 == 1;
    // Every load here is a round trip to the coherence point (about a microsecond),
    // so a merge takes one: a merge takes at most kMaxMerge partials (the host's
    // grouping), whose maxima and sums go to LDS while each thread loads its
    // elements' accumulators of every partial.  The partials are merged in split
    // (or group) order, each weighted by exp2(m_i - M) under the overall maximum M.
    constexpr int NE = (GQ * D + kThreads - 1) / kThreads;  // (head, channel) elements per thread
    __shared__ float2 s_pml[kMaxMerge * GQ];
    int hk[NE], ck[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = min(tid + k * kThreads, GQ * D - 1);
        hk[k] = e / D;
        ck[k] = e % D;
    }
    for (;;) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = prev == (unsigned)(ns - 1);
        }
        __syncthreads();
        if (!*s_last) return;
        // The merge, with NB >= ns partials' loads per element (the power of two
        // above ns): loads beyond ns repeat the last partial's addresses, and each is
        // a round trip of its own to the coherence point, so they are not padded to
        // kMaxMerge.
        auto merge = [&](auto nbc) __attribute__((always_inline)) {
            constexpr int NB = decltype(nbc)::value;
            constexpr int NPB = (NB * GQ + kThreads - 1) / kThreads;  // (partial, head) pairs per thread
            const int npair = ns * GQ;
            float2 mlr[NPB];
#pragma unroll
            for (int r = 0; r < NPB; ++r) mlr[r] = fetch2(&pml[2 * min(tid + r * kThreads, npair - 1)]);
            float ai[NE][NB];
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int k = 0; k < NE; ++k) ai[k][i] = fetch(&pacc[(min(i, ns - 1) * GQ + hk[k]) * D + ck[k]]);
#pragma unroll
            for (int r = 0; r < NPB; ++r)
                if (tid + r * kThreads < npair) s_pml[tid + r * kThreads] = mlr[r];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                float M = -INFINITY, L = 0.0f, A = 0.0f;
                for (int i = 0; i < ns; ++i) M = fmaxf(M, s_pml[i * GQ + hk[k]].x);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    if (i < ns) {
                        const float2 ml = s_pml[i * GQ + hk[k]];
                        const float w = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - M);
                        L = fmaf(ml.y, w, L);
                        A = fmaf(ai[k][i], w, A);
                    }
                }
                if (tid + k * kThreads >= GQ * D) continue;
                const int h = hk[k], c = ck[k];
                if (final) {
                    a.out[(qrow0 + h) * D + c] = A / L;
                    if (c == 0 && a.lse) a.lse[qrow0 + h] = (M + __log2f(L)) * 0.69314718055994530942f;
                } else {
                    // this group's partial
                    const int64_t gidx = (bh * a.cgroups_cap + grp) * GQ + h;
                    publish(&a.grp_acc[gidx * D + c], A);
                    if (c == 0) {
                        publish(&a.grp_ml[gidx * 2], M);
                        publish(&a.grp_ml[gidx * 2 + 1], L);
                    }
                }
            }
        };
        static_assert(kMaxMerge == 16, "merge sizes 2, 4, 8, 16");
        if (ns <= 2) merge(std::integral_constant<int, 2>());
        else if (ns <= 4) merge(std::integral_constant<int, 4>());
        else if (ns <= 8) merge(std::integral_constant<int, 8>());
        else merge(std::integral_constant<int, 16>());
        // this counter's arrivals are all counted: clear it for the next call
        if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (final) return;
        // second level: this group's partial is published; count it at the slice
        pml = a.grp_ml + bh * a.cgroups_cap * GQ * 2;
        pacc = a.grp_acc + bh * a.cgroups_cap * GQ * D;
        ns = ng1;
        ctr = a.counters + bh;
        final = true;
    }
}

}  // namespace dec
}  // namespace kvq
