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
//     the split streams groups w, w+4, ... tile by tile, one tile ahead;
//   - keys: a token row is spread over LPT = D / CPL lanes (CPL codes each), so a
//     wave scores TPW = 64 / LPT tokens per load; the per-lane integer partials
//     are summed over the LPT lanes with DPP;
//   - values: dword (block, channel) of the value codes holds one channel of TB
//     consecutive tokens; a lane owns D/32 channels of one block, so its value
//     dot products run along tokens;
//   - softmax weights and digits move between the two mappings through LDS as
//     bytes, and are packed into digit dwords with one shift-or;
//   - the running max is wave-uniform and updated once per tile;
//   - sinks and residual tokens (full precision) are spread over the splits and
//     scored with fp32 FMAs through the same state;
//   - all GQ query heads that share a kv head run in the same workgroup, so each
//     KV byte is read from HBM once.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace dec {

struct DecArgs {
    const uint8_t* rec;  // key-group records
    const char* ksink;
    const char* vsink;
    const char* kres;
    const char* vres;
    const void* q;
    float* out;
    float* lse;
    float* part_acc;     // [BH][nsplit_cap][GQ][D]
    float* part_ml;      // [BH][nsplit_cap][GQ][2]
    unsigned* counters;  // [BH]
    int64_t ng_cap;
    int rec_bytes, rec_kcodes, rec_vcodes, rec_vmeta;
    int Hkv, S, R, nS, nfp, G, GV, nvg, log2nvg, gps, ngroups, nsplit, nsplit_cap;
    float qscale;  // sm_scale * log2(e)
};

constexpr int kLimbs = 5;
constexpr float kLazy = 8.0f;  // running-max slack (log2 units) before a rescale

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes; every lane of a group gets the
// same (bitwise identical) sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (N >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Max over aligned groups of N consecutive lanes (same pattern as group_sum).
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
    if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Max over the slots of a wave when every group of LPT lanes holds one value:
// reduces lanes LPT apart (values are equal inside a group).
template <int LPT>
__device__ __forceinline__ float slots_max(float v) {
    if constexpr (LPT == 1) return group_max<64>(v);
    else if constexpr (LPT == 2) { v = fmaxf(v, dpp<0x4E>(v)); }
    if constexpr (LPT <= 4) v = fmaxf(v, dpp<0x141>(v));
    if constexpr (LPT <= 8) v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// max / sum over all lanes whose index agrees modulo `from` (a power of two)
__device__ __forceinline__ float xor_max(float v, int from) {
    for (int off = from; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float xor_sum(float v, int from) {
    for (int off = from; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
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

// balanced base-16 digits of n (|n| <= 2^18): digit i as a two's-complement nibble
__device__ __forceinline__ void store_digits(uint8_t* dst, int stride, int n) {
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) {
        dst[i * stride] = (uint8_t)(n & 15);
        n = (n + 8) >> 4;
    }
}

__device__ __forceinline__ uint32_t lds32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// A nibble dword of codes pairs a "lo" run of 4 items (byte k, low nibble) with a
// "hi" run of 4 items (byte k, high nibble); the matching digit dword is built
// from the two runs of digit bytes.
__device__ __forceinline__ uint32_t digit_dword(const uint8_t* lo, const uint8_t* hi) {
    return lds32(lo) | (lds32(hi) << 4);
}

template <int N>
__device__ __forceinline__ float pick(const float (&a)[N], int i) {
    float r = a[0];
#pragma unroll
    for (int k = 1; k < N; ++k) r = (i == k) ? a[k] : r;
    return r;
}

template <int DT, int N>
__device__ __forceinline__ void load_row(const char* base, int64_t elem0, float (&f)[N]) {
#pragma unroll
    for (int c = 0; c < N; ++c) f[c] = load_as_f32<DT>(base, elem0 + c);
}

template <int LW>
struct Vec;
template <>
struct Vec<1> {
    using T = uint32_t;
};
template <>
struct Vec<2> {
    using T = uint2;
};
template <>
struct Vec<4> {
    using T = uint4;
};

template <int LW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t (&w)[LW]) {
    using T = typename Vec<LW>::T;
    T v = *reinterpret_cast<const T*>(p);
    __builtin_memcpy(w, &v, sizeof(T));
}

// ---------------------------------------------------------------------------
// LDS carve-up (dynamic shared memory)
// ---------------------------------------------------------------------------
template <int D, int GQ, int TILE>
struct LdsPlan {
    // per wave: key digits [GQ][limb][D] bytes, weight digits [GQ][nvg][limb][TILE]
    // bytes, weight scales [GQ][nvg] fp32
    __host__ __device__ static int wave_bytes(int nvg) {
        const int b = GQ * kLimbs * D + GQ * nvg * kLimbs * TILE + 4 * GQ * nvg;
        return (b + 15) & ~15;
    }
    // per workgroup: wave states and combine scratch
    __host__ __device__ static int wg_floats() { return kWaves * GQ * D + kWaves * GQ * 2 + kMaxCombine + 16 + 4; }
    __host__ __device__ static int bytes(int nvg) { return kWaves * wave_bytes(nvg) + 4 * wg_floats(); }
};

// ---------------------------------------------------------------------------
// the kernel: grid = (nsplit, BH)
// ---------------------------------------------------------------------------
template <int DT, int BITS, int D, int GQ, int CPL, int TILE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecArgs a) {
    constexpr int LPT = D / CPL;           // key lanes per token
    constexpr int TPW = 64 / LPT;          // tokens per key wave-load
    constexpr int U = TILE / TPW;          // tokens per slot per tile
    constexpr int LW = CPL * BITS / 32;    // packed key dwords per lane per token
    constexpr int KND = CPL / 8;           // key nibble dwords per lane per token
    constexpr int RB = D * BITS / 8;       // key row bytes
    constexpr int TB = 32 / BITS;          // tokens per value dword
    constexpr int VCPL = D / 32;           // value channels per lane
    constexpr int NVL = TILE / (2 * TB);   // value wave-loads per tile
    constexpr int VNE = TB / 8;            // nibble dwords per value code dword
    constexpr int KM = D / 64;             // channels per lane in the query fold
    constexpr int ZB = BITS == 4 ? 8 : 0;  // code bias
    static_assert(LW >= 1 && LW * 32 == CPL * BITS, "key lane chunk must be whole dwords");
    static_assert(U >= 1 && U * TPW == TILE, "tile must be whole key wave-loads");
    static_assert(NVL >= 1 && NVL * 2 * TB == TILE, "tile must be whole value wave-loads");

    extern __shared__ __align__(16) unsigned char dsm[];
    using LP = LdsPlan<D, GQ, TILE>;

    const int split = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int b = (int)(bh / a.Hkv), kvh = (int)(bh % a.Hkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nvg = a.nvg;

    uint8_t* kd = dsm + wave * LP::wave_bytes(nvg);            // key digits
    uint8_t* pd = kd + GQ * kLimbs * D;                         // weight digits
    float* psc = reinterpret_cast<float*>(pd + GQ * nvg * kLimbs * TILE);
    float* wg = reinterpret_cast<float*>(dsm + kWaves * LP::wave_bytes(nvg));
    float* s_acc = wg;                                          // [kWaves][GQ][D]
    float* s_ml = s_acc + kWaves * GQ * D;                      // [kWaves][GQ][2]
    float* s_cw = s_ml + kWaves * GQ * 2;                       // [kMaxCombine]
    float* s_cM = s_cw + kMaxCombine;                           // [8]
    float* s_cL = s_cM + 8;                                     // [8]
    int* s_last = reinterpret_cast<int*>(s_cL + 8);

    const int slot = lane / LPT, chunk = lane % LPT;
    const int hb = lane >> 5;                  // value half: block parity
    const int c0v = (lane & 31) * VCPL;        // value channels of this lane
    const int gv = c0v / a.GV;                 // their value group
    const int gz = chunk & (nvg - 1);          // value group of this lane's (token, group) pairs
    const int64_t qrow0 = (int64_t)b * a.Hkv * GQ + (int64_t)kvh * GQ;

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
    auto update_max = [&](const float (&mt)[GQ]) {
        bool grow = false;
        float mnew[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            mnew[h] = fmaxf(m[h], mt[h]);
            grow |= mnew[h] > m[h];
        }
        if (grow) {  // wave-uniform
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
    const int G = a.G;
    const int tpg = G / TILE;
    const int g_begin = split * a.gps;
    const int g_end = min(g_begin + a.gps, a.ngroups);
    const int n_my_groups = g_begin + wave < g_end ? (g_end - g_begin - wave + kWaves - 1) / kWaves : 0;
    const int n_tiles = n_my_groups * tpg;

    if (n_tiles > 0) {
        float qv[GQ][KM];
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int j = 0; j < KM; ++j)
                qv[h][j] = load_as_f32<DT>(a.q, (qrow0 + h) * D + KM * lane + j) * a.qscale;

        // One tile of this wave's stream; ks/kz are the key scales/zeros of the
        // tile's group, loaded when the tile is the first of its group.
        struct Tile {
            uint32_t k[U][LW];
            uint32_t v[NVL][VCPL];
            float2 vm[U];
            float ks[KM], kz[KM];
        };
        // Loader position: record of the current group and tile within it.  Once the
        // last tile has been issued, further loads repeat it (never out of range).
        const uint8_t* lrec = a.rec + rec_offset(bh, g_begin + wave, a.ng_cap, a.rec_bytes);
        const size_t group_step = (size_t)kWaves * a.rec_bytes;
        int ltig = 0, issued = 0;
        const int upairs = U * nvg;
        auto load_next = [&](Tile& t) {
            const uint8_t* r = lrec;
            const int t0 = ltig * TILE;  // first token of the tile in its group
#pragma unroll
            for (int u = 0; u < U; ++u)
                load_words<LW>(r + a.rec_kcodes + (t0 + u * TPW + slot) * RB + chunk * (LW * 4), t.k[u]);
#pragma unroll
            for (int vl = 0; vl < NVL; ++vl)
                load_words<VCPL>(r + a.rec_vcodes + ((size_t)(t0 / TB + 2 * vl + hb) * D + c0v) * 4, t.v[vl]);
            const float* vmeta = reinterpret_cast<const float*>(r + a.rec_vmeta);
#pragma unroll
            for (int k = 0; k < U; ++k) {
                int p = chunk + k * LPT;
                p = p < upairs ? p : chunk;  // unused pairs reload a valid one
                t.vm[k] = *reinterpret_cast<const float2*>(
                    vmeta + ((t0 + (p >> a.log2nvg) * TPW + slot) * nvg + gz) * 2);
            }
            if (ltig == 0) {  // wave-uniform
                const float* km = reinterpret_cast<const float*>(r);
#pragma unroll
                for (int j = 0; j < KM; ++j) t.ks[j] = km[KM * lane + j], t.kz[j] = km[D + KM * lane + j];
            }
            if (issued + 1 < n_tiles) {
                ++issued;
                if (++ltig == tpg) {
                    ltig = 0;
                    lrec += group_step;
                }
            }
        };

        uint32_t kl[GQ][kLimbs][KND];  // key digit dwords of this lane's channels
        float kinv[GQ], kbias[GQ];
        int ctig = 0;  // consumer: tile within group

        // Value accumulators in fixed point: per channel and digit, sums of
        // dot8(weight digits, codes - 8) over all tiles since the last flush; they
        // represent accv += vinv * sum_i 16^i va[i].  Each dot8 is at most 512 in
        // magnitude, so they cannot overflow within a split.
        int va[GQ][VCPL][kLimbs];
        float vmul[GQ], vinv[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            vmul[h] = 0.0f;
            vinv[h] = 0.0f;
#pragma unroll
            for (int c = 0; c < VCPL; ++c)
#pragma unroll
                for (int li = 0; li < kLimbs; ++li) va[h][c][li] = 0;
        }
        auto flush_head = [&](int h) {
            const float w1 = vinv[h] * 16.0f, w2 = vinv[h] * 256.0f, w3 = vinv[h] * 4096.0f,
                        w4 = vinv[h] * 65536.0f;
#pragma unroll
            for (int c = 0; c < VCPL; ++c) {
                float t = accv[h][c];
                t = fmaf((float)va[h][c][0], vinv[h], t);
                t = fmaf((float)va[h][c][1], w1, t);
                t = fmaf((float)va[h][c][2], w2, t);
                t = fmaf((float)va[h][c][3], w3, t);
                t = fmaf((float)va[h][c][4], w4, t);
                accv[h][c] = t;
#pragma unroll
                for (int li = 0; li < kLimbs; ++li) va[h][c][li] = 0;
            }
        };

        auto process = [&](const Tile& cur) {
            if (ctig == 0) {
                // fold the group's key scales into the query, in fixed point
                float qt[GQ][KM], mx[GQ], bp[GQ];
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    mx[h] = 0.0f;
                    bp[h] = 0.0f;
#pragma unroll
                    for (int j = 0; j < KM; ++j) {
                        qt[h][j] = qv[h][j] * cur.ks[j];
                        mx[h] = fmaxf(mx[h], fabsf(qt[h][j]));
                        bp[h] = fmaf(qt[h][j], cur.kz[j] - (float)ZB, bp[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const FixScale fs = fix_scale(group_max<64>(mx[h]));
                    kinv[h] = fs.inv;
                    kbias[h] = group_sum<64>(bp[h]);
#pragma unroll
                    for (int j = 0; j < KM; ++j)
                        store_digits(kd + (h * kLimbs) * D + KM * lane + j, D, (int)rintf(qt[h][j] * fs.mul));
                }
                wave_lds_sync();
#pragma unroll
                for (int h = 0; h < GQ; ++h)
#pragma unroll
                    for (int li = 0; li < kLimbs; ++li) {
                        const uint8_t* base = kd + (h * kLimbs + li) * D + chunk * CPL;
#pragma unroll
                        for (int nd = 0; nd < KND; ++nd) {
                            if constexpr (BITS == 4)
                                kl[h][li][nd] = digit_dword(base + 8 * nd, base + 8 * nd + 4);
                            else
                                kl[h][li][nd] = digit_dword(base + 16 * (nd >> 1) + 4 * (nd & 1),
                                                            base + 16 * (nd >> 1) + 8 + 4 * (nd & 1));
                        }
                    }
                wave_lds_sync();
            }
            if (++ctig == tpg) ctig = 0;

            // ---- key scores of this slot's U tokens ----
            float sc[GQ][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t cw[KND];
#pragma unroll
                for (int d = 0; d < LW; ++d) {
                    if constexpr (BITS == 4) {
                        cw[d] = cur.k[u][d] ^ 0x88888888u;
                    } else {
                        cw[2 * d] = cur.k[u][d] & 0x33333333u;
                        cw[2 * d + 1] = (cur.k[u][d] >> 2) & 0x33333333u;
                    }
                }
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    int acc = 0;
#pragma unroll
                    for (int li = kLimbs - 1; li >= 0; --li) {
                        acc <<= 4;
#pragma unroll
                        for (int nd = 0; nd < KND; ++nd) acc = dot8(kl[h][li][nd], cw[nd], acc);
                    }
                    sc[h][u] = (float)acc;
                }
            }
            // ---- online softmax, lazily rescaled: the running max only moves when
            //      a tile's max exceeds it by more than kLazy (weights stay <= 2^kLazy)
            float mt[GQ];
            bool grow = false;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                mt[h] = -INFINITY;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    sc[h][u] = group_sum<LPT>(sc[h][u]) * kinv[h] - kbias[h];
                    mt[h] = fmaxf(mt[h], sc[h][u]);
                }
                mt[h] = slots_max<LPT>(mt[h]);
                grow |= mt[h] > m[h] + kLazy;
            }
            bool rescaled[GQ];
#pragma unroll
            for (int h = 0; h < GQ; ++h) rescaled[h] = false;
            if (grow) {  // wave-uniform
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    if (mt[h] > m[h] + kLazy) {
                        flush_head(h);
                        const float f = fast_exp2(m[h] - mt[h]);
                        m[h] = mt[h];
                        lpart[h] *= f;
                        zpart[h] *= f;
#pragma unroll
                        for (int c = 0; c < VCPL; ++c) accv[h][c] *= f;
                        rescaled[h] = true;
                    }
                }
            }

            // ---- weights p_t s_t -> fixed-point digits in LDS ----
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float p[U];
#pragma unroll
                for (int u = 0; u < U; ++u) p[u] = fast_exp2(sc[h][u] - m[h]);
                float pt[U], mx = 0.0f;
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int pi = chunk + k * LPT;
                    const bool valid = pi < upairs;
                    const float pu = pick(p, pi >> a.log2nvg);
                    pt[k] = valid ? pu * cur.vm[k].x : 0.0f;
                    zpart[h] = fmaf(pt[k], cur.vm[k].y - (float)ZB, zpart[h]);
                    if (valid && gz == 0) lpart[h] += pu;
                    mx = fmaxf(mx, pt[k]);
                }
                mx = group_max<64>(mx);
                // keep the fixed-point scale unless this tile would overflow it
                if (rescaled[h] || mx * vmul[h] >= 262144.0f) {  // wave-uniform
                    if (!rescaled[h]) flush_head(h);
                    const FixScale fs = fix_scale(mx);
                    vmul[h] = fs.mul;
                    vinv[h] = fs.inv;
                }
                uint8_t* dst = pd + ((h * nvg + gz) * kLimbs) * TILE;
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int pi = chunk + k * LPT;
                    if (pi < upairs)
                        store_digits(dst + (pi >> a.log2nvg) * TPW + slot, TILE, (int)rintf(pt[k] * vmul[h]));
                }
            }
            wave_lds_sync();

            // ---- values: dot products along tokens into the fixed-point accumulators ----
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const uint8_t* pbase = pd + ((h * nvg + gv) * kLimbs) * TILE;
#pragma unroll
                for (int vl = 0; vl < NVL; ++vl) {
                    const int blk = 2 * vl + hb;  // block within the tile
                    uint32_t vw[VCPL][VNE];
#pragma unroll
                    for (int c = 0; c < VCPL; ++c) {
                        if constexpr (BITS == 4) {
                            vw[c][0] = cur.v[vl][c] ^ 0x88888888u;
                        } else {
                            vw[c][0] = cur.v[vl][c] & 0x33333333u;
                            vw[c][VNE - 1] = (cur.v[vl][c] >> 2) & 0x33333333u;
                        }
                    }
#pragma unroll
                    for (int li = 0; li < kLimbs; ++li) {
                        const uint8_t* tb = pbase + li * TILE + blk * TB;
                        uint32_t dl[VNE];
                        if constexpr (BITS == 4) {
                            dl[0] = digit_dword(tb, tb + 4);
                        } else {
                            dl[0] = digit_dword(tb, tb + 8);
                            dl[VNE - 1] = digit_dword(tb + 4, tb + 12);
                        }
#pragma unroll
                        for (int c = 0; c < VCPL; ++c)
#pragma unroll
                            for (int e = 0; e < VNE; ++e) va[h][c][li] = dot8(dl[e], vw[c][e], va[h][c][li]);
                    }
                }
            }
            wave_lds_sync();
        };

        // three tile buffers: two tiles in flight while one is processed
        Tile t0, t1, t2;
        load_next(t0);
        load_next(t1);
        for (int i = 0; i < n_tiles; i += 3) {
            load_next(t2);
            process(t0);
            if (i + 1 >= n_tiles) break;
            load_next(t0);
            process(t1);
            if (i + 2 >= n_tiles) break;
            load_next(t1);
            process(t2);
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) flush_head(h);
    }

    // ---------------- full-precision tokens (sinks, residual) ----------------
    const int f0 = (int)((int64_t)split * a.nfp / a.nsplit);
    const int f1 = (int)((int64_t)(split + 1) * a.nfp / a.nsplit);
    if (f1 > f0) {
        float qf[GQ][CPL];
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                qf[h][c] = load_as_f32<DT>(a.q, (qrow0 + h) * D + chunk * CPL + c) * a.qscale;
        auto row_of = [&](int j, const char*& kp, const char*& vp) -> int64_t {
            if (j < a.nS) {
                kp = a.ksink, vp = a.vsink;
                return bh * a.S + j;
            }
            kp = a.kres, vp = a.vres;
            return bh * a.R + (j - a.nS);
        };
        for (int j0 = f0 + wave * TPW; j0 < f1; j0 += kWaves * TPW) {
            const int j = j0 + slot;
            const bool valid = j < f1;
            float s[GQ];
            {
                float kf[CPL];
                const char *kp, *vp;
                const int64_t row = row_of(valid ? j : f0, kp, vp);
                load_row<DT, CPL>(kp, row * D + chunk * CPL, kf);
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    float t = 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) t = fmaf(qf[h][c], kf[c], t);
                    t = group_sum<LPT>(t);
                    s[h] = valid ? t : -INFINITY;
                }
            }
            float mt[GQ];
#pragma unroll
            for (int h = 0; h < GQ; ++h) mt[h] = xor_max(s[h], LPT);
            update_max(mt);
            float pv[GQ];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                pv[h] = valid ? fast_exp2(s[h] - m[h]) : 0.0f;
                if (chunk == 0) lpart[h] += pv[h];
            }
            // value rows: half hb takes slots hb, hb + 2, ...
            for (int k = 0; k < TPW / 2; ++k) {
                const int sl = 2 * k + hb;
                float psl[GQ];
#pragma unroll
                for (int h = 0; h < GQ; ++h) psl[h] = __shfl(pv[h], sl * LPT);
                const int jt = j0 + sl;
                if (jt < f1) {
                    const char *kp, *vp;
                    const int64_t row = row_of(jt, kp, vp);
                    float vf[VCPL];
                    load_row<DT, VCPL>(vp, row * D + c0v, vf);
#pragma unroll
                    for (int h = 0; h < GQ; ++h)
#pragma unroll
                        for (int c = 0; c < VCPL; ++c) accv[h][c] = fmaf(psl[h], vf[c], accv[h][c]);
                }
            }
        }
    }

    // ---------------- wave state -> LDS ----------------
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        const float L = xor_sum(lpart[h], 1);
        const float Zg = xor_sum(zpart[h], nvg);  // total for value group lane % nvg
        const float Zv = __shfl(Zg, gv);
#pragma unroll
        for (int c = 0; c < VCPL; ++c) {
            const float tot = accv[h][c] + __shfl_xor(accv[h][c], 32) - Zv;
            if (lane < 32) s_acc[(wave * GQ + h) * D + c0v + c] = tot;
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

    // Last workgroup of this slice merges all splits (log-sum-exp combine).
    // The partials were written with device-scope stores, which write through the
    // XCD's L2; every wave waits until its stores are acknowledged, then one
    // thread counts the arrival.  The last arrival reads the partials back with
    // device-scope loads.  No L2 write-back or invalidate is needed because all
    // data exchanged between workgroups moves through device-scope accesses.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(&a.counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = prev == (unsigned)(a.nsplit - 1);
    }
    __syncthreads();
    if (!*s_last) return;

    const int ns = a.nsplit;
    const float* pml = a.part_ml + bh * a.nsplit_cap * GQ * 2;
    const float* pacc = a.part_acc + bh * a.nsplit_cap * GQ * D;
    // per-head max and weights over splits: head h handled by wave h % kWaves
    for (int h = wave; h < GQ; h += kWaves) {
        float M = -INFINITY;
        for (int i = lane; i < ns; i += 64) M = fmaxf(M, fetch(&pml[(i * GQ + h) * 2]));
        M = xor_max(M, 1);
        float L = 0.0f;
        for (int i = lane; i < ns; i += 64) {
            const float mi = fetch(&pml[(i * GQ + h) * 2]);
            const float li = fetch(&pml[(i * GQ + h) * 2 + 1]);
            const float w = (mi == -INFINITY) ? 0.0f : fast_exp2(mi - M);
            s_cw[i * GQ + h] = w;
            L = fmaf(li, w, L);
        }
        L = group_sum<64>(L);
        if (lane == 0) {
            s_cM[h] = M;
            s_cL[h] = L;
        }
    }
    __syncthreads();
    for (int e = tid; e < GQ * D; e += kThreads) {
        const int h = e / D, c = e % D;
        float A0 = 0.0f, A1 = 0.0f, A2 = 0.0f, A3 = 0.0f;
        int i = 0;
        for (; i + 4 <= ns; i += 4) {
            A0 = fmaf(fetch(&pacc[((i + 0) * GQ + h) * D + c]), s_cw[(i + 0) * GQ + h], A0);
            A1 = fmaf(fetch(&pacc[((i + 1) * GQ + h) * D + c]), s_cw[(i + 1) * GQ + h], A1);
            A2 = fmaf(fetch(&pacc[((i + 2) * GQ + h) * D + c]), s_cw[(i + 2) * GQ + h], A2);
            A3 = fmaf(fetch(&pacc[((i + 3) * GQ + h) * D + c]), s_cw[(i + 3) * GQ + h], A3);
        }
        for (; i < ns; ++i) A0 = fmaf(fetch(&pacc[(i * GQ + h) * D + c]), s_cw[i * GQ + h], A0);
        const float L = s_cL[h];
        a.out[(qrow0 + h) * D + c] = ((A0 + A1) + (A2 + A3)) / L;
        if (c == 0 && a.lse) a.lse[qrow0 + h] = (s_cM[h] + __log2f(L)) * 0.69314718055994530942f;
    }
    if (tid == 0) __hip_atomic_store(&a.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dec
}  // namespace kvq
