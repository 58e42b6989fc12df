// decode_impl.h -- split-token decode attention over the low-bit KV cache (gfx950).
//
// out = softmax(q K'^T * sm_scale) V' over sinks, quantized tokens and residual
// ("KV Cache的Int4量化：如何解决Attention Sink导致的量化精度崩塌问题", section 3;
// KIVI notes "LLM系列：KVCache量化1 KIVI…", section 1: the logits of the grouped
// part and of the residual are concatenated before one softmax).  Token order
// does not matter ("Resumo Técnico: LogQuant", Metodologia 4), so the token
// range of every (sequence, kv head) slice is cut into splits that run in
// parallel; each split keeps an online-softmax state (running max m, sum l,
// unnormalised accumulator) and the states are merged with a log-sum-exp
// combine by the last workgroup of the slice to finish.
//
// Mapping on CDNA4 (wave64):
//   - one workgroup = 4 waves = one split; waves take interleaved key groups;
//   - a token row of packed codes is spread over LPT = D / CPL lanes, each lane
//     loading CPL codes (4..16 bytes) of K and of V per token: a wave streams
//     TPW = 64 / LPT tokens per load instruction, fully coalesced;
//   - key scale/zero are folded into the query once per key group:
//       q . k' = sum_c (q_c s_c) code_c - sum_c (q_c s_c) z_c
//     (the identity behind the zero-point cross terms of "Atom…", section 三
//     "核心公式"), so the inner loop is one FMA per code per query head;
//     q_c s_c is built in LDS by the whole wave and read back per lane;
//   - the value scale/zero fold the same way into the softmax weight:
//       sum_j p_j v'_jc = sum_j (p_j s_j) code_jc - sum_j (p_j s_j) z_j;
//   - per-token dot products are reduced over the LPT lanes with DPP
//     (quad_perm, row_half_mirror, row_mirror); the softmax runs in base 2 with
//     log2(e) folded into the query, one max update per tile of TILE tokens;
//   - all GQ query heads sharing a kv head are served by the same workgroup, so
//     every KV byte is read from HBM once.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace dec {

struct DecArgs {
    const uint8_t* kcodes;
    const uint8_t* vcodes;
    const float* kmeta;
    const float* vmeta;
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
    int64_t Lq_cap, ng_cap, Lq;
    int Hkv, S, R, nS, r, G, GV, nvg, gps, nsplit_q, nsplit, nsplit_cap, has_fp;
    float qscale;  // sm_scale * log2(e)
};

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// device-scope store / load of split partials exchanged between workgroups
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// codes of LW packed dwords -> floats in channel order
template <int BITS, int LW>
__device__ __forceinline__ void unpack(const uint32_t (&w)[LW], float (&f)[LW * (32 / BITS)]) {
    constexpr int CPD = 32 / BITS;
    constexpr uint32_t MASK = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
#pragma unroll
    for (int d = 0; d < LW; ++d) {
#pragma unroll
        for (int sub = 0; sub < CPD / 4; ++sub) {
            // opaque mask so that each byte converts with one v_cvt_f32_ubyteN
            uint32_t x;
            asm("v_and_b32 %0, %1, %2" : "=v"(x) : "i"(MASK), "v"(w[d] >> (BITS * sub)));
            f[d * CPD + 4 * sub + 0] = (float)(x & 0xFFu);
            f[d * CPD + 4 * sub + 1] = (float)((x >> 8) & 0xFFu);
            f[d * CPD + 4 * sub + 2] = (float)((x >> 16) & 0xFFu);
            f[d * CPD + 4 * sub + 3] = (float)(x >> 24);
        }
    }
}

// ---------------------------------------------------------------------------
// shared memory of one workgroup
// ---------------------------------------------------------------------------
template <int D, int GQ>
struct Smem {
    float qt[kWaves][GQ][D];       // folded query per wave
    float acc[kWaves][GQ][D];      // per-wave merged accumulators
    float ml[kWaves][GQ][2];       // per-wave (m, l)
    float cw[kMaxCombine];         // combine weights
    float cM[8], cL[8];
    int last;
};

// Merge the per-slot states of a wave (slots = groups of LPT lanes) and store the
// wave's state in shared memory.  acc holds the lane's N channels chunk*N.. of
// every head; m, l are per slot.
template <int D, int GQ, int LPT, int N>
__device__ __forceinline__ void wave_state_to_lds(Smem<D, GQ>& sm, float (&m)[GQ], float (&l)[GQ],
                                                  float (&acc)[GQ][N], int lane, int wave) {
    const int chunk = lane % LPT;
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = (M == -INFINITY) ? 0.0f : fast_exp2(m[h] - M);
        float lh = l[h] * f;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) lh += __shfl_xor(lh, off);
#pragma unroll
        for (int c = 0; c < N; ++c) {
            float a = acc[h][c] * f;
#pragma unroll
            for (int off = LPT; off < 64; off <<= 1) a += __shfl_xor(a, off);
            acc[h][c] = a;
        }
        if (lane < LPT) {
#pragma unroll
            for (int c = 0; c < N; ++c) sm.acc[wave][h][chunk * N + c] = acc[h][c];
            if (lane == 0) {
                sm.ml[wave][h][0] = M;
                sm.ml[wave][h][1] = lh;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// quantized split: key groups [g_begin, g_end) of slice bh
// ---------------------------------------------------------------------------
template <int DT, int BITS, int D, int GQ, int CPL, int TILE>
__device__ __forceinline__ void quant_split(const DecArgs& a, Smem<D, GQ>& sm, int64_t bh, int b,
                                            int kvh, int split, int lane, int wave) {
    constexpr int LPT = D / CPL;
    constexpr int TPW = 64 / LPT;
    constexpr int LB = CPL * BITS / 8;
    constexpr int LW = LB / 4;
    constexpr int RB = D * BITS / 8;
    constexpr int U = TILE / TPW;
    constexpr int KM = D / 64;  // channels per lane when folding the query
    static_assert(LW >= 1 && LW * 4 == LB, "lane chunk must be whole dwords");
    static_assert(U >= 1 && U * TPW == TILE, "tile must be whole wave loads");

    const int slot = lane / LPT;
    const int chunk = lane % LPT;
    const int G = a.G;
    const int tpg = G / TILE;

    const int g_begin = split * a.gps;
    int g_end = g_begin + a.gps;
    const int ng = (int)(a.Lq / G);
    if (g_end > ng) g_end = ng;
    const int n_my_groups = (g_end - g_begin - wave + kWaves - 1) / kWaves;
    const int n_tiles = n_my_groups > 0 ? n_my_groups * tpg : 0;

    // query (pre-scaled by sm_scale * log2 e) for this lane's KM folding channels
    float qv[GQ][KM];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int j = 0; j < KM; ++j)
            qv[h][j] = load_as_f32<DT>(a.q, ((int64_t)b * a.Hkv * GQ + (int64_t)kvh * GQ + h) * D +
                                                KM * lane + j) * a.qscale;

    float m[GQ], l[GQ], zacc[GQ], bias[GQ];
    float acc[GQ][CPL];
    float qt[GQ][CPL];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
        zacc[h] = 0.0f;
        bias[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[h][c] = 0.0f, qt[h][c] = 0.0f;
    }

    const uint8_t* kbase = a.kcodes + bh * a.Lq_cap * RB + chunk * LB;
    const uint8_t* vbase = a.vcodes + bh * a.Lq_cap * RB + chunk * LB;
    const float* vmbase = a.vmeta + (bh * a.Lq_cap * a.nvg + (chunk * CPL) / a.GV) * 2;
    const float* kmbase = a.kmeta + bh * a.ng_cap * 2 * D + KM * lane;

    struct Tile {
        uint32_t k[U][LW];
        uint32_t v[U][LW];
        float2 vm[U];
    };
    auto tile_token0 = [&](int i) -> int64_t {
        const int grp = g_begin + wave + (i / tpg) * kWaves;
        return (int64_t)grp * G + (int64_t)(i % tpg) * TILE + slot;
    };
    auto load_tile = [&](int i, Tile& t) {
        const int64_t tok0 = tile_token0(i);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tok = tok0 + u * TPW;
            load_words<LW>(kbase + tok * RB, t.k[u]);
            load_words<LW>(vbase + tok * RB, t.v[u]);
            t.vm[u] = *reinterpret_cast<const float2*>(vmbase + tok * a.nvg * 2);
        }
    };
    struct KMeta {
        float s[KM], z[KM];
    };
    auto load_kmeta = [&](int i, KMeta& km) {
        const int grp = g_begin + wave + (i / tpg) * kWaves;
        const float* p = kmbase + (int64_t)grp * 2 * D;
#pragma unroll
        for (int j = 0; j < KM; ++j) km.s[j] = p[j], km.z[j] = p[D + j];
    };

    if (n_tiles > 0) {
        Tile cur;
        KMeta kmc;
        load_kmeta(0, kmc);
        load_tile(0, cur);
        for (int i = 0; i < n_tiles; ++i) {
            Tile nxt;
            KMeta kmn = kmc;
            const int inext = i + 1 < n_tiles ? i + 1 : i;
            if ((i + 1) % tpg == 0 && i + 1 < n_tiles) load_kmeta(i + 1, kmn);
            load_tile(inext, nxt);

            if (i % tpg == 0) {
                // fold this group's key scales into the query; bias = sum_c qt_c z_c
                float bp[GQ];
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    bp[h] = 0.0f;
#pragma unroll
                    for (int j = 0; j < KM; ++j) {
                        const float t = qv[h][j] * kmc.s[j];
                        sm.qt[wave][h][KM * lane + j] = t;
                        bp[h] = fmaf(t, kmc.z[j], bp[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < GQ; ++h) bias[h] = group_sum<64>(bp[h]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int h = 0; h < GQ; ++h)
#pragma unroll
                    for (int c = 0; c < CPL; c += 4) {
                        const float4 t = *reinterpret_cast<const float4*>(&sm.qt[wave][h][chunk * CPL + c]);
                        qt[h][c] = t.x, qt[h][c + 1] = t.y, qt[h][c + 2] = t.z, qt[h][c + 3] = t.w;
                    }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }

            // scores of the U tokens of this slot
            float sc[GQ][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[CPL];
                unpack<BITS, LW>(cur.k[u], kf);
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    float s = 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) s = fmaf(qt[h][c], kf[c], s);
                    sc[h][u] = s;
                }
            }
            bool grow = false;
            float mnew[GQ];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float mt = -INFINITY;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    sc[h][u] = group_sum<LPT>(sc[h][u]) - bias[h];
                    mt = fmaxf(mt, sc[h][u]);
                }
                mnew[h] = fmaxf(m[h], mt);
                grow |= mnew[h] > m[h];
            }
            if (__any(grow)) {
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const float f = fast_exp2(m[h] - mnew[h]);
                    m[h] = mnew[h];
                    l[h] *= f;
                    zacc[h] *= f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[h][c] *= f;
                }
            }
            // values
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[CPL];
                unpack<BITS, LW>(cur.v[u], vf);
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const float p = fast_exp2(sc[h][u] - m[h]);
                    l[h] += p;
                    const float pt = p * cur.vm[u].x;
                    zacc[h] = fmaf(pt, cur.vm[u].y, zacc[h]);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[h][c] = fmaf(pt, vf[c], acc[h][c]);
                }
            }
            cur = nxt;
            kmc = kmn;
        }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[h][c] -= zacc[h];
    wave_state_to_lds<D, GQ, LPT, CPL>(sm, m, l, acc, lane, wave);
}

// ---------------------------------------------------------------------------
// full-precision split: sinks and residual of slice bh
// ---------------------------------------------------------------------------
template <int DT, int D, int GQ>
__device__ __forceinline__ void fp_split(const DecArgs& a, Smem<D, GQ>& sm, int64_t bh, int b, int kvh,
                                         int lane, int wave) {
    constexpr int LPT = 16;
    constexpr int N = D / LPT;  // channels per lane
    constexpr int TPW = 64 / LPT;
    const int slot = lane / LPT;
    const int chunk = lane % LPT;
    const int T = a.nS + a.r;

    float qf[GQ][N];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int c = 0; c < N; ++c)
            qf[h][c] = load_as_f32<DT>(a.q, ((int64_t)b * a.Hkv * GQ + (int64_t)kvh * GQ + h) * D +
                                                chunk * N + c) * a.qscale;
    float m[GQ], l[GQ], acc[GQ][N];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < N; ++c) acc[h][c] = 0.0f;
    }
    for (int j0 = wave * TPW; j0 < T; j0 += kWaves * TPW) {
        const int j = j0 + slot;
        if (j < T) {
            const char* kp;
            const char* vp;
            int64_t row;
            if (j < a.nS) {
                kp = a.ksink, vp = a.vsink, row = bh * a.S + j;
            } else {
                kp = a.kres, vp = a.vres, row = bh * a.R + (j - a.nS);
            }
            float kf[N], vf[N];
#pragma unroll
            for (int c = 0; c < N; ++c) {
                kf[c] = load_as_f32<DT>(kp, row * D + chunk * N + c);
                vf[c] = load_as_f32<DT>(vp, row * D + chunk * N + c);
            }
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float s = 0.0f;
#pragma unroll
                for (int c = 0; c < N; ++c) s = fmaf(qf[h][c], kf[c], s);
                s = group_sum<LPT>(s);
                const float mn = fmaxf(m[h], s);
                const float f = fast_exp2(m[h] - mn);
                const float p = fast_exp2(s - mn);
                m[h] = mn;
                l[h] = l[h] * f + p;
#pragma unroll
                for (int c = 0; c < N; ++c) acc[h][c] = fmaf(p, vf[c], acc[h][c] * f);
            }
        }
    }
    wave_state_to_lds<D, GQ, LPT, N>(sm, m, l, acc, lane, wave);
}

// ---------------------------------------------------------------------------
// the kernel: grid = (nsplit, BH); split nsplit_q (if present) is full precision
// ---------------------------------------------------------------------------
template <int DT, int BITS, int D, int GQ, int CPL, int TILE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecArgs a) {
    __shared__ Smem<D, GQ> sm;
    const int split = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int b = (int)(bh / a.Hkv), kvh = (int)(bh % a.Hkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (split < a.nsplit_q)
        quant_split<DT, BITS, D, GQ, CPL, TILE>(a, sm, bh, b, kvh, split, lane, wave);
    else
        fp_split<DT, D, GQ>(a, sm, bh, b, kvh, lane, wave);
    __syncthreads();

    // merge the waves of this workgroup
    const int64_t qrow0 = (int64_t)b * a.Hkv * GQ + (int64_t)kvh * GQ;  // first query head row
    const bool single = a.nsplit == 1;
    for (int e = tid; e < GQ * D; e += kThreads) {
        const int h = e / D, c = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.ml[w][h][0]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm.ml[w][h][0];
            const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
            L = fmaf(sm.ml[w][h][1], f, L);
            A = fmaf(sm.acc[w][h][c], f, A);
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
        sm.last = prev == (unsigned)(a.nsplit - 1);
    }
    __syncthreads();
    if (!sm.last) return;

    const int ns = a.nsplit;
    const float* pml = a.part_ml + bh * a.nsplit_cap * GQ * 2;
    const float* pacc = a.part_acc + bh * a.nsplit_cap * GQ * D;
    // per-head max and sum over splits: head h handled by wave h % kWaves
    for (int h = wave; h < GQ; h += kWaves) {
        float M = -INFINITY;
        for (int i = lane; i < ns; i += 64) M = fmaxf(M, fetch(&pml[(i * GQ + h) * 2]));
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        float L = 0.0f;
        for (int i = lane; i < ns; i += 64) {
            const float mi = fetch(&pml[(i * GQ + h) * 2]);
            const float li = fetch(&pml[(i * GQ + h) * 2 + 1]);
            const float w = (mi == -INFINITY) ? 0.0f : fast_exp2(mi - M);
            sm.cw[i * GQ + h] = w;
            L = fmaf(li, w, L);
        }
        L = group_sum<64>(L);
        if (lane == 0) {
            sm.cM[h] = M;
            sm.cL[h] = L;
        }
    }
    __syncthreads();
    for (int e = tid; e < GQ * D; e += kThreads) {
        const int h = e / D, c = e % D;
        float A0 = 0.0f, A1 = 0.0f, A2 = 0.0f, A3 = 0.0f;
        int i = 0;
        for (; i + 4 <= ns; i += 4) {
            A0 = fmaf(fetch(&pacc[((i + 0) * GQ + h) * D + c]), sm.cw[(i + 0) * GQ + h], A0);
            A1 = fmaf(fetch(&pacc[((i + 1) * GQ + h) * D + c]), sm.cw[(i + 1) * GQ + h], A1);
            A2 = fmaf(fetch(&pacc[((i + 2) * GQ + h) * D + c]), sm.cw[(i + 2) * GQ + h], A2);
            A3 = fmaf(fetch(&pacc[((i + 3) * GQ + h) * D + c]), sm.cw[(i + 3) * GQ + h], A3);
        }
        for (; i < ns; ++i) A0 = fmaf(fetch(&pacc[(i * GQ + h) * D + c]), sm.cw[i * GQ + h], A0);
        const float L = sm.cL[h];
        a.out[(qrow0 + h) * D + c] = ((A0 + A1) + (A2 + A3)) / L;
        if (c == 0 && a.lse) a.lse[qrow0 + h] = (sm.cM[h] + __log2f(L)) * 0.69314718055994530942f;
    }
    if (tid == 0) __hip_atomic_store(&a.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dec
}  // namespace kvq
