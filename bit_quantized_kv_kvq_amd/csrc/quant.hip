// quant.hip -- append, flush (group quantize + pack), dequantize and export kernels.
//
// Group quantizer (asymmetric min-max, "Atom: Low-bit Quantization for Efficient
// and Accurate LLM Serving", section 三 "核心公式"; dequantization from "KV Cache的
// Int4量化：如何解决Attention Sink导致的量化精度崩塌问题", section 2):
//   s = (max - min) / (2^n - 1); z = rint(-min / s); q = clamp(rint(x / s) + z, 0, 2^n - 1)
//   x' = (q - z) * s
// binary32 with one rounding per operation in this order (IEEE division, rint =
// round half to even); a zero scale (constant group or underflowing range) is
// replaced by |min| (1 when min == 0); a zero point of -0 is stored as +0.
// Grouping (KIVI notes, "LLM系列：KVCache量化1 KIVI…", section 1): keys per channel
// over each run of G tokens, values per token over each run of G_V channels.
// Flushes: the whole residual when it reaches R tokens (KIVI notes, section 1),
// or, under log-sparse retention ("Resumo Técnico: LogQuant", Metodologia
// item 2), the earlier token of each pair among the oldest 2W of a residual of
// R = 3W tokens, the later ones and the newest W staying at full precision.
#include <algorithm>

#include "kvq_internal.h"

namespace kvq {
namespace {

#pragma clang fp contract(off)

struct QParams {
    float s, z;
};

__device__ inline QParams group_params(float mn, float mx, float qmax) {
    float range = mx - mn;
    float s = range / qmax;
    if (mx == mn || s == 0.0f) s = (mn != 0.0f) ? fabsf(mn) : 1.0f;
    float z = rintf((-mn) / s);
    if (z == 0.0f) z = 0.0f;  // +0
    return {s, z};
}

// Symmetric variant: s = 2 max|x| / (2^n - 1), z = 2^(n-1) (the signed code
// clamp(round(x / s), -2^(n-1), 2^(n-1) - 1) plus 2^(n-1) is group_code's
// clamp(round(x / s) + z, 0, 2^n - 1): both sides are exact small integers).
__device__ inline QParams group_params_sym(float mn, float mx, float qmax) {
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    float s = (2.0f * amax) / qmax;
    if (s == 0.0f) s = (amax != 0.0f) ? amax : 1.0f;
    return {s, 0.5f * (qmax + 1.0f)};
}

__device__ inline uint32_t group_code(float x, QParams p, float qmax) {
    float t = rintf(x / p.s) + p.z;
    t = t < 0.0f ? 0.0f : t;
    t = t > qmax ? qmax : t;
    return (uint32_t)t;
}

// ---------------------------------------------------------------------------
// token copy (sink / residual slots), 16-byte vectors
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_tokens_kernel(const uint4* __restrict__ src_k,
                                                          const uint4* __restrict__ src_v,
                                                          int64_t src_tokens, int64_t src_tok0,
                                                          uint4* __restrict__ dst_k,
                                                          uint4* __restrict__ dst_v, int64_t dst_tokens,
                                                          int64_t dst_tok0, int64_t n, int row_vec,
                                                          int64_t bh0, int64_t total) {
    // total = nbh * n * row_vec vectors of K, then as many of V
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const bool is_v = i >= total;
        const int64_t j = is_v ? i - total : i;
        const int64_t v = j % row_vec;
        const int64_t t = (j / row_vec) % n;
        const int64_t bh = bh0 + j / ((int64_t)row_vec * n);
        const int64_t si = (bh * src_tokens + src_tok0 + t) * row_vec + v;
        const int64_t di = (bh * dst_tokens + dst_tok0 + t) * row_vec + v;
        if (is_v)
            dst_v[di] = src_v[si];
        else
            dst_k[di] = src_k[si];
    }
}

// One token per sequence (src [BH][D]) into each slice's own sink slot or residual
// row, for caches whose sequences differ in length: the slice's length before the
// append is base_len[b] + delta.  A slice with n < S tokens takes sink slot n;
// otherwise residual row n - S - Lq (fewer than R tokens wait there).
__global__ __launch_bounds__(256) void copy_one_ragged_kernel(const uint4* __restrict__ src_k,
                                                              const uint4* __restrict__ src_v,
                                                              uint4* __restrict__ ksink, uint4* __restrict__ vsink,
                                                              uint4* __restrict__ kres, uint4* __restrict__ vres,
                                                              const int* __restrict__ base_len, int delta,
                                                              int Hkv, int S, int R, int Qf, int row_vec,
                                                              int64_t total) {
    // total = BH * row_vec vectors of K, then as many of V
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const bool is_v = i >= total;
        const int64_t j = is_v ? i - total : i;
        const int64_t v = j % row_vec;
        const int64_t bh = j / row_vec;
        const int64_t n = (int64_t)base_len[bh / Hkv] + delta;
        const SliceState st = slice_state(n, S, R, Qf);
        uint4* dst;
        if (n < S) dst = (is_v ? vsink : ksink) + (bh * S + n) * row_vec + v;
        else dst = (is_v ? vres : kres) + (bh * R + st.r) * row_vec + v;
        *dst = (is_v ? src_v : src_k)[bh * row_vec + v];
    }
}

// Log-sparse retention, after the flush has quantized residual rows 0, 2, ...,
// 2W - 2: rows 1, 3, ..., 2W - 1 move to rows 0 .. W - 1 and rows 2W .. 3W - 1
// to rows W .. 2W - 1, in place.  Row i takes row 2i + 1 (i < W) or i + W
// (i >= W), always a row above i, so a thread that moves one 16-byte column of
// a slice in increasing i never reads a row it has already overwritten; loading
// a run of kRun source rows before storing them is safe for the same reason
// (rows written by earlier runs lie below the run).
constexpr int kRun = 8;
__global__ __launch_bounds__(256) void log_compact_kernel(uint4* kres, uint4* vres, int R, int W, int row_vec,
                                                          int64_t bh0, int64_t total) {
    // total = nbh * row_vec columns of K, then as many of V
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const bool is_v = i >= total;
        const int64_t j = is_v ? i - total : i;
        const int64_t bh = bh0 + j / row_vec;
        uint4* col = (is_v ? vres : kres) + bh * R * row_vec + j % row_vec;
        for (int i0 = 0; i0 < 2 * W; i0 += kRun) {
            uint4 x[kRun];
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                const int r = i0 + u;
                x[u] = col[(int64_t)(r < W ? 2 * r + 1 : r + W) * row_vec];
            }
#pragma unroll
            for (int u = 0; u < kRun; ++u) col[(int64_t)(i0 + u) * row_vec] = x[u];
        }
    }
}

// dst[idx[i]] = val[i] for i < n (entries passed in the kernel arguments)
constexpr int kEntryChunk = 256;
struct EntryChunk {
    int n;
    int idx[kEntryChunk];
    int val[kEntryChunk];
};
__global__ __launch_bounds__(kEntryChunk) void set_entries_kernel(int* __restrict__ dst, EntryChunk c) {
    if ((int)threadIdx.x < c.n) dst[c.idx[threadIdx.x]] = c.val[threadIdx.x];
}

// base_len[i] = v[i] for i < n (values passed in the kernel arguments)
constexpr int kLenChunk = 256;
struct LenChunk {
    int n;
    int v[kLenChunk];
};
__global__ __launch_bounds__(kLenChunk) void set_lengths_kernel(int* __restrict__ dst, LenChunk c) {
    if ((int)threadIdx.x < c.n) dst[threadIdx.x] = c.v[threadIdx.x];
}

// ---------------------------------------------------------------------------
// quantize + pack one key group (G tokens x D channels) and the values of the
// same G tokens into the group's record.  grid = (n_groups, BH), block = 256.
// ---------------------------------------------------------------------------
struct QuantArgs {
    const void* src_k;
    const void* src_v;
    int64_t src_tokens, src_tok0, dst_tok0;
    int tok_stride;  // source rows between consecutive tokens (2: every other row)
    int D, G, GV, nvg, row_bytes;
    int64_t ng_cap;
    int rec_bytes, rec_kcodes, rec_vcodes, rec_vmeta;
    int codec;     // kvq_codec
    int key_axis;  // kvq_key_axis
    int64_t bh0;   // first slice of the launch
    RecMap rm;
    int outliers, rec_kov, rec_koi, rec_vov, rec_voi;  // dense-and-sparse records
};

// The larger of two (magnitude, index) candidates, the lower index among equal
// magnitudes: the outlier rule of dense-and-sparse groups.
__device__ inline void outlier_max(float& m, int& i, float m2, int i2) {
    if (m2 > m || (m2 == m && i2 < i)) m = m2, i = i2;
}

// key rows: dword w of token row t holds channels CPD*w + j at pack_shift(j)
// (each field biased by code_bias)
template <int BITS>
__device__ inline void pack_rows(const uint8_t* s_codes, int rows, int D, int row_bytes,
                                 uint8_t* dst_row0) {
    constexpr int CPD = 32 / BITS;  // channels per dword
    const int dpr = D / CPD;
    for (int i = threadIdx.x; i < rows * dpr; i += blockDim.x) {
        int t = i / dpr, w = i % dpr;
        const uint8_t* c = s_codes + t * D + w * CPD;
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < CPD; ++j) word |= ((uint32_t)c[j] ^ code_bias(BITS)) << pack_shift(BITS, j);
        reinterpret_cast<uint32_t*>(dst_row0 + (int64_t)t * row_bytes)[w] = word;
    }
}

// value blocks: dword (b, c) holds tokens TB*b + j of channel c at pack_shift(j)
// (each field biased by code_bias)
template <int BITS>
__device__ inline void pack_blocks(const uint8_t* s_codes, int rows, int D, uint32_t* dst) {
    constexpr int TB = 32 / BITS;  // tokens per dword
    const int nblk = rows / TB;
    for (int i = threadIdx.x; i < nblk * D; i += blockDim.x) {
        const int b = i / D, c = i % D;
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < TB; ++j)
            word |= ((uint32_t)s_codes[(b * TB + j) * D + c] ^ code_bias(BITS)) << pack_shift(BITS, j);
        dst[i] = word;
    }
}

// Storage words of 8 consecutive elements (16 bytes of a 16-bit dtype, 32 bytes
// of fp32) as fp32.
template <int DT>
__device__ inline void load8_f32(const void* base, int64_t elem0, float (&f)[8]) {
    if constexpr (DT == DT_F32) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem0);
        const float4 x = p[0], y = p[1];
        f[0] = x.x, f[1] = x.y, f[2] = x.z, f[3] = x.w, f[4] = y.x, f[5] = y.y, f[6] = y.z, f[7] = y.w;
    } else {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t lo = (uint16_t)(ws[i] & 0xFFFFu), hi = (uint16_t)(ws[i] >> 16);
            f[2 * i] = DT == DT_BF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
            f[2 * i + 1] = DT == DT_BF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
        }
    }
}

// Two consecutive elements as fp32.
template <int DT>
__device__ inline void load2_f32(const void* base, int64_t elem0, float& x0, float& x1) {
    if constexpr (DT == DT_F32) {
        const float2 x = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + elem0);
        x0 = x.x, x1 = x.y;
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + elem0);
        const uint16_t lo = (uint16_t)(w & 0xFFFFu), hi = (uint16_t)(w >> 16);
        x0 = DT == DT_BF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
        x1 = DT == DT_BF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
}

// Per-token groups: for each of the G tokens of a key group, one group per run of
// GV channels (nvg = D / GV groups per token), quantized into s_codes ([G][D]
// bytes) with (scale, zero) in meta [G][nvg][2].  TPI consecutive lanes share one
// (token, group), each with GV/TPI channels in runs of 8 (16-byte loads), and
// meet by lane shuffles.  Values always; keys too under per-token keys (GV = D).
// sp_rec: the record whose value-outlier fields take dense-and-sparse outliers
// (null: no outliers).
template <int DT, int BITS>
__device__ inline void token_groups(const QuantArgs& a, const void* src, int64_t src_row0, int GV, int nvg,
                                    float* meta, uint8_t* s_codes, uint8_t* sp_rec) {
    constexpr float qmax = (float)((1 << BITS) - 1);
    const int D = a.D, G = a.G, tid = threadIdx.x, ts = a.tok_stride;
    const bool sparse = sp_rec != nullptr;
    const int items = G * nvg;
    int tpi = 256 / items;                    // lanes per (token, group)
    tpi = tpi < 1 ? 1 : tpi > GV / 8 ? GV / 8 : tpi;
    const int cpt = GV / tpi;                 // channels per lane, a multiple of 8
    for (int i0 = 0; i0 < items * tpi; i0 += 256) {
        const int i = (i0 + tid) / tpi, sub = (i0 + tid) % tpi;
        const bool live = i < items;
        const int t = live ? i / nvg : 0, h = live ? i % nvg : 0;
        const int64_t e0 = (src_row0 + (int64_t)t * ts) * D + (int64_t)h * GV + sub * cpt;
        // outliers: channel (within the group) of largest magnitude
        int ov = -1;
        if (sparse) {
            float am = -1.0f;
            int ai = 0;
            for (int j = 0; j < cpt; j += 8) {
                float f[8];
                load8_f32<DT>(src, e0 + j, f);
#pragma unroll
                for (int k = 0; k < 8; ++k) outlier_max(am, ai, fabsf(f[k]), sub * cpt + j + k);
            }
            for (int m = 1; m < tpi; m <<= 1)   // lanes of one item are consecutive
                outlier_max(am, ai, __shfl_xor(am, m), __shfl_xor(ai, m));
            ov = ai;
        }
        float mn = INFINITY, mx = -INFINITY;
        for (int j = 0; j < cpt; j += 8) {
            float f[8];
            load8_f32<DT>(src, e0 + j, f);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (sub * cpt + j + k != ov) mn = fminf(mn, f[k]), mx = fmaxf(mx, f[k]);
        }
        for (int o = 1; o < tpi; o <<= 1) {   // lanes of one item are consecutive
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        const QParams p = a.codec ? group_params_sym(mn, mx, qmax) : group_params(mn, mx, qmax);
        if (live) {
            for (int j = 0; j < cpt; j += 8) {
                float f[8];
                load8_f32<DT>(src, e0 + j, f);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo |= group_code(f[k], p, qmax) << (8 * k);
                    hi |= group_code(f[k + 4], p, qmax) << (8 * k);
                }
                *reinterpret_cast<uint2*>(s_codes + t * D + h * GV + sub * cpt + j) = make_uint2(lo, hi);
            }
            if (sub == 0) {
                meta[i * 2] = p.s;
                meta[i * 2 + 1] = p.z;
            }
            if (sparse && ov >= sub * cpt && ov < (sub + 1) * cpt) {
                const float x = load_as_f32<DT>(src, e0 - sub * cpt + ov);
                reinterpret_cast<float*>(sp_rec + a.rec_vov)[i] = x;
                reinterpret_cast<uint16_t*>(sp_rec + a.rec_voi)[i] = (uint16_t)(ov | (group_code(x, p, qmax) << 8));
            }
        }
    }
}

// One workgroup per key group.  Keys: thread (channel pair cp, part p) covers
// tokens [p G/P, (p+1) G/P) of channels 2cp, 2cp+1 (coalesced across the
// workgroup); the P partial minima/maxima of a channel meet in LDS.  Values: TPI
// consecutive lanes share one (token, value group), each with GV/TPI channels in
// runs of 8 (16-byte loads), and meet by lane shuffles.  Every element is read
// twice (min/max, then codes); the second read hits the caches.  Codes go to LDS
// and are packed from there.  Per-token keys take the values' path with one group
// per token over D channels.  Dense-and-sparse groups first find each vector's
// outlier (largest magnitude, lowest index among equals; KVQuant, per-vector
// dense-and-sparse quantization) the same way, leave it out of the min/max, and
// store its exact value, place and code beside the record.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr float qmax = (float)((1 << BITS) - 1);
    const int grp = blockIdx.x;
    const int64_t bh = a.bh0 + blockIdx.y;
    const int D = a.D, G = a.G, tid = threadIdx.x;
    uint8_t* s_codes = smem;                                               // [G][D]
    float* s_mm = reinterpret_cast<float*>(smem + (((size_t)G * D + 15) & ~(size_t)15));  // [P][D][2]
    const int ts = a.tok_stride;
    const int64_t src_row0 = bh * a.src_tokens + a.src_tok0 + (int64_t)grp * G * ts;
    const int64_t dst_grp = a.dst_tok0 / G + grp;
    uint8_t* rec = rec_ptr(a.rm, bh, dst_grp);
    float* kmeta = reinterpret_cast<float*>(rec);

    // ---- keys ----
    if (a.key_axis == 1) {
        // per token: one group over the token's D channels ("Atom…" review, section
        // 三, model-components table, KV-cache row: attention-head granularity)
        token_groups<DT, BITS>(a, a.src_k, src_row0, D, 1, kmeta, s_codes, nullptr);
    } else {
        const int CH = D / 2;            // channel pairs
        const int P = 256 / CH;          // token parts (4 for D = 128, 8 for D = 64)
        const int GP = G / P;            // tokens per thread
        const int cp = tid % CH, part = tid / CH, c = 2 * cp;
        const int64_t e0 = (src_row0 + (int64_t)part * GP * ts) * D + c;
        const int64_t sD = (int64_t)ts * D;
        // outliers: token of largest magnitude of each of the two channels
        int o0 = -1, o1 = -1;
        if (a.outliers) {
            float a0 = -1.0f, a1 = -1.0f;
            int i0 = 0, i1 = 0;
            for (int t = 0; t < GP; ++t) {
                float x0, x1;
                load2_f32<DT>(a.src_k, e0 + t * sD, x0, x1);
                outlier_max(a0, i0, fabsf(x0), part * GP + t);
                outlier_max(a1, i1, fabsf(x1), part * GP + t);
            }
            s_mm[(part * D + c) * 2] = a0, s_mm[(part * D + c) * 2 + 1] = __int_as_float(i0);
            s_mm[(part * D + c + 1) * 2] = a1, s_mm[(part * D + c + 1) * 2 + 1] = __int_as_float(i1);
            __syncthreads();
            a0 = s_mm[c * 2], i0 = __float_as_int(s_mm[c * 2 + 1]);
            a1 = s_mm[(c + 1) * 2], i1 = __float_as_int(s_mm[(c + 1) * 2 + 1]);
            for (int q = 1; q < P; ++q) {
                outlier_max(a0, i0, s_mm[(q * D + c) * 2], __float_as_int(s_mm[(q * D + c) * 2 + 1]));
                outlier_max(a1, i1, s_mm[(q * D + c + 1) * 2], __float_as_int(s_mm[(q * D + c + 1) * 2 + 1]));
            }
            o0 = i0 - part * GP, o1 = i1 - part * GP;  // in this thread's run, or outside it
            __syncthreads();
        }
        float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll 8
        for (int t = 0; t < GP; ++t) {
            float x0, x1;
            load2_f32<DT>(a.src_k, e0 + t * sD, x0, x1);
            if (t != o0) mn0 = fminf(mn0, x0), mx0 = fmaxf(mx0, x0);
            if (t != o1) mn1 = fminf(mn1, x1), mx1 = fmaxf(mx1, x1);
        }
        s_mm[(part * D + c) * 2] = mn0, s_mm[(part * D + c) * 2 + 1] = mx0;
        s_mm[(part * D + c + 1) * 2] = mn1, s_mm[(part * D + c + 1) * 2 + 1] = mx1;
        __syncthreads();
        mn0 = s_mm[c * 2], mx0 = s_mm[c * 2 + 1], mn1 = s_mm[(c + 1) * 2], mx1 = s_mm[(c + 1) * 2 + 1];
        for (int q = 1; q < P; ++q) {
            mn0 = fminf(mn0, s_mm[(q * D + c) * 2]), mx0 = fmaxf(mx0, s_mm[(q * D + c) * 2 + 1]);
            mn1 = fminf(mn1, s_mm[(q * D + c + 1) * 2]), mx1 = fmaxf(mx1, s_mm[(q * D + c + 1) * 2 + 1]);
        }
        const QParams p0 = a.codec ? group_params_sym(mn0, mx0, qmax) : group_params(mn0, mx0, qmax);
        const QParams p1 = a.codec ? group_params_sym(mn1, mx1, qmax) : group_params(mn1, mx1, qmax);
#pragma unroll 8
        for (int t = 0; t < GP; ++t) {
            float x0, x1;
            load2_f32<DT>(a.src_k, e0 + t * sD, x0, x1);
            const uint32_t q0 = group_code(x0, p0, qmax), q1 = group_code(x1, p1, qmax);
            *reinterpret_cast<uint16_t*>(s_codes + (part * GP + t) * D + c) = (uint16_t)(q0 | (q1 << 8));
        }
        if (part == 0) {
            kmeta[c] = p0.s, kmeta[c + 1] = p1.s;
            kmeta[D + c] = p0.z, kmeta[D + c + 1] = p1.z;
        }
        // the outliers' exact values, token and code: by the thread whose run holds them
        if (a.outliers) {
            float* kov = reinterpret_cast<float*>(rec + a.rec_kov);
            uint16_t* koi = reinterpret_cast<uint16_t*>(rec + a.rec_koi);
            if (o0 >= 0 && o0 < GP) {
                float x0, x1;
                load2_f32<DT>(a.src_k, e0 + o0 * sD, x0, x1);
                kov[c] = x0;
                koi[c] = (uint16_t)((part * GP + o0) | (group_code(x0, p0, qmax) << 8));
            }
            if (o1 >= 0 && o1 < GP) {
                float x0, x1;
                load2_f32<DT>(a.src_k, e0 + o1 * sD, x0, x1);
                kov[c + 1] = x1;
                koi[c + 1] = (uint16_t)((part * GP + o1) | (group_code(x1, p1, qmax) << 8));
            }
        }
    }
    __syncthreads();
    pack_rows<BITS>(s_codes, G, D, a.row_bytes, rec + a.rec_kcodes);
    __syncthreads();

    // ---- values ----
    token_groups<DT, BITS>(a, a.src_v, src_row0, a.GV, a.nvg, reinterpret_cast<float*>(rec + a.rec_vmeta), s_codes,
                           a.outliers ? rec : nullptr);
    __syncthreads();
    pack_blocks<BITS>(s_codes, G, D, reinterpret_cast<uint32_t*>(rec + a.rec_vcodes));
}

// ---------------------------------------------------------------------------
// dequantize to fp32 in token order (sinks, quantized, residual)
// ---------------------------------------------------------------------------
struct DeqArgs {
    const char* ksink;
    const char* vsink;
    const char* kres;
    const char* vres;
    RecMap rm;
    float* kout;
    float* vout;
    int64_t nS, Lq, r, T, ng_cap;  // the slices' state; with base_len, the longest sequence's
    int S, R, Qf, D, G, GV, nvg, bits, row_bytes;
    int rec_bytes, rec_kcodes, rec_vcodes, rec_vmeta;
    const int* base_len;  // sequences of different lengths (see Ragged), or null
    int delta;
    int Hkv;
    int outliers, rec_kov, rec_koi, rec_vov, rec_voi;  // dense-and-sparse records
    int key_axis;  // kvq_key_axis: key (scale, zero) [2][D], or [G][2] per token
};

// State of slice bh: the launch's (uniform) one, or the one of its sequence's length.
__device__ inline void deq_slice(const DeqArgs& a, int64_t bh, int64_t& nS, int64_t& Lq, int64_t& r) {
    nS = a.nS, Lq = a.Lq, r = a.r;
    if (a.base_len != nullptr) {
        const SliceState st = slice_state((int64_t)a.base_len[bh / a.Hkv] + a.delta, a.S, a.R, a.Qf);
        nS = st.nS, Lq = st.Lq, r = st.r;
    }
}

__device__ inline uint32_t key_code(const DeqArgs& a, const uint8_t* rec, int t, int c) {
    const int cpd = 32 / a.bits;
    const uint32_t w = reinterpret_cast<const uint32_t*>(rec + a.rec_kcodes + (int64_t)t * a.row_bytes)[c / cpd];
    return ((w >> pack_shift(a.bits, c % cpd)) & ((1u << a.bits) - 1u)) ^ code_bias(a.bits);
}

__device__ inline uint32_t value_code(const DeqArgs& a, const uint8_t* rec, int t, int c) {
    const int tb = 32 / a.bits;
    const uint32_t w = reinterpret_cast<const uint32_t*>(rec + a.rec_vcodes)[(t / tb) * a.D + c];
    return ((w >> pack_shift(a.bits, t % tb)) & ((1u << a.bits) - 1u)) ^ code_bias(a.bits);
}

template <int DT>
__global__ __launch_bounds__(256) void dequantize_kernel(DeqArgs a) {
    const int64_t bh = blockIdx.y;
    int64_t nS, Lq, r;
    deq_slice(a, bh, nS, Lq, r);
    const int64_t n = (nS + Lq + r) * a.D;  // this slice's tokens; rows up to a.T in the output
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / a.D;
        const int c = (int)(i % a.D);
        float kx, vx;
        if (t < nS) {
            const int64_t idx = (bh * a.S + t) * a.D + c;
            kx = load_as_f32<DT>(a.ksink, idx);
            vx = load_as_f32<DT>(a.vsink, idx);
        } else if (t < nS + Lq) {
            const int64_t tq = t - nS;
            const int tg = (int)(tq % a.G);
            const uint8_t* rec = rec_ptr(a.rm, bh, tq / a.G);
            const float* km = reinterpret_cast<const float*>(rec);
            const float* vm = reinterpret_cast<const float*>(rec + a.rec_vmeta) + ((int64_t)tg * a.nvg + c / a.GV) * 2;
            const float kq = (float)key_code(a, rec, tg, c);
            const float vq = (float)value_code(a, rec, tg, c);
            const float ks = a.key_axis ? km[2 * tg] : km[c];
            const float kz = a.key_axis ? km[2 * tg + 1] : km[a.D + c];
            kx = (kq - kz) * ks;
            vx = (vq - vm[1]) * vm[0];
            if (a.outliers) {  // outliers dequantize to their exact values
                if ((reinterpret_cast<const uint16_t*>(rec + a.rec_koi)[c] & 0xFF) == tg)
                    kx = reinterpret_cast<const float*>(rec + a.rec_kov)[c];
                const int item = tg * a.nvg + c / a.GV;
                if ((reinterpret_cast<const uint16_t*>(rec + a.rec_voi)[item] & 0xFF) == c % a.GV)
                    vx = reinterpret_cast<const float*>(rec + a.rec_vov)[item];
            }
        } else {
            const int64_t idx = (bh * a.R + (t - nS - Lq)) * a.D + c;
            kx = load_as_f32<DT>(a.kres, idx);
            vx = load_as_f32<DT>(a.vres, idx);
        }
        a.kout[(bh * a.T + t) * a.D + c] = kx;
        a.vout[(bh * a.T + t) * a.D + c] = vx;
    }
}

// ---------------------------------------------------------------------------
// canonical export of codes and metadata
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void export_kernel(DeqArgs a, uint8_t* k_codes, float* k_scale,
                                                     float* k_zero, uint8_t* v_codes,
                                                     float* v_scale, float* v_zero) {
    const int64_t bh = blockIdx.y;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t nS_b, Lq_b, r_b;
    deq_slice(a, bh, nS_b, Lq_b, r_b);
    const int64_t ncode = a.Lq * a.D;  // output rows per slice (the longest sequence's)
    for (int64_t i = i0; i < Lq_b * a.D; i += stride) {
        const int64_t t = i / a.D;
        const int c = (int)(i % a.D);
        const uint8_t* rec = rec_ptr(a.rm, bh, t / a.G);
        const int tg = (int)(t % a.G);
        if (k_codes) k_codes[bh * ncode + i] = (uint8_t)key_code(a, rec, tg, c);
        if (v_codes) v_codes[bh * ncode + i] = (uint8_t)value_code(a, rec, tg, c);
    }
    if (a.key_axis) {   // per token: [Lq][1]
        for (int64_t t = i0; t < Lq_b; t += stride) {
            const float* km = reinterpret_cast<const float*>(rec_ptr(a.rm, bh, t / a.G)) + 2 * (t % a.G);
            if (k_scale) k_scale[bh * a.Lq + t] = km[0];
            if (k_zero) k_zero[bh * a.Lq + t] = km[1];
        }
    } else {
        const int64_t nk = (a.Lq / a.G) * a.D;
        for (int64_t i = i0; i < (Lq_b / a.G) * a.D; i += stride) {
            const int64_t g = i / a.D;
            const int c = (int)(i % a.D);
            const float* km = reinterpret_cast<const float*>(rec_ptr(a.rm, bh, g));
            if (k_scale) k_scale[bh * nk + i] = km[c];
            if (k_zero) k_zero[bh * nk + i] = km[a.D + c];
        }
    }
    const int64_t nv = a.Lq * a.nvg;
    for (int64_t i = i0; i < Lq_b * a.nvg; i += stride) {
        const int64_t t = i / a.nvg;
        const int h = (int)(i % a.nvg);
        const uint8_t* rec = rec_ptr(a.rm, bh, t / a.G);
        const float* vm = reinterpret_cast<const float*>(rec + a.rec_vmeta) + ((t % a.G) * a.nvg + h) * 2;
        if (v_scale) v_scale[bh * nv + i] = vm[0];
        if (v_zero) v_zero[bh * nv + i] = vm[1];
    }
}

// The outliers of dense-and-sparse records: key outliers' token within the group
// and exact value [BH][Lq/G][D], value outliers' channel within the group and
// exact value [BH][Lq][nvg] (rows up to the longest sequence's; a shorter
// slice's rows past its own are not written).
__global__ __launch_bounds__(256) void export_outliers_kernel(DeqArgs a, uint8_t* k_idx, float* k_val,
                                                              uint8_t* v_idx, float* v_val) {
    const int64_t bh = blockIdx.y;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t nS_b, Lq_b, r_b;
    deq_slice(a, bh, nS_b, Lq_b, r_b);
    const int64_t nk = (a.Lq / a.G) * a.D;
    for (int64_t i = i0; i < (Lq_b / a.G) * a.D; i += stride) {
        const uint8_t* rec = rec_ptr(a.rm, bh, i / a.D);
        const int c = (int)(i % a.D);
        if (k_idx) k_idx[bh * nk + i] = (uint8_t)(reinterpret_cast<const uint16_t*>(rec + a.rec_koi)[c] & 0xFF);
        if (k_val) k_val[bh * nk + i] = reinterpret_cast<const float*>(rec + a.rec_kov)[c];
    }
    const int64_t nv = a.Lq * a.nvg;
    for (int64_t i = i0; i < Lq_b * a.nvg; i += stride) {
        const int64_t t = i / a.nvg;
        const uint8_t* rec = rec_ptr(a.rm, bh, t / a.G);
        const int item = (int)((t % a.G) * a.nvg + i % a.nvg);
        if (v_idx) v_idx[bh * nv + i] = (uint8_t)(reinterpret_cast<const uint16_t*>(rec + a.rec_voi)[item] & 0xFF);
        if (v_val) v_val[bh * nv + i] = reinterpret_cast<const float*>(rec + a.rec_vov)[item];
    }
}

DeqArgs make_deq_args(const Layout& L, const DevPtrs& P, int64_t nS, int64_t Lq, int64_t r, Ragged rg) {
    DeqArgs a;
    a.key_axis = L.key_axis;
    a.outliers = L.outliers;
    a.rec_kov = L.rec_kov;
    a.rec_koi = L.rec_koi;
    a.rec_vov = L.rec_vov;
    a.rec_voi = L.rec_voi;
    a.base_len = rg.base_len;
    a.delta = rg.delta;
    a.Hkv = L.Hkv;
    a.ksink = P.ksink;
    a.vsink = P.vsink;
    a.kres = P.kres;
    a.vres = P.vres;
    a.rm = rec_map(L, P);
    a.kout = nullptr;
    a.vout = nullptr;
    a.nS = nS;
    a.Lq = Lq;
    a.r = r;
    a.T = nS + Lq + r;
    a.ng_cap = L.ng_cap;
    a.S = L.S;
    a.R = L.R;
    a.Qf = L.Qf;
    a.D = L.D;
    a.G = L.G;
    a.GV = L.GV;
    a.nvg = L.nvg;
    a.bits = L.bits;
    a.row_bytes = L.row_bytes;
    a.rec_bytes = L.rec_bytes;
    a.rec_kcodes = L.rec_kcodes;
    a.rec_vcodes = L.rec_vcodes;
    a.rec_vmeta = L.rec_vmeta;
    return a;
}

int grid_for(int64_t work, int64_t per_block, int cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

hipError_t launch_copy_tokens(const Layout& L, const void* src_k, const void* src_v,
                              int64_t src_tokens, int64_t src_tok0, char* dst_k, char* dst_v,
                              int64_t dst_tokens, int64_t dst_tok0, int64_t n, int64_t bh0, int64_t nbh,
                              hipStream_t stream) {
    if (n <= 0 || nbh <= 0) return hipSuccess;
    const int row_vec = L.D * L.esize / 16;
    const int64_t total = nbh * n * row_vec;
    const int grid = grid_for(2 * total, 256, 65535);
    copy_tokens_kernel<<<grid, 256, 0, stream>>>(
        reinterpret_cast<const uint4*>(src_k), reinterpret_cast<const uint4*>(src_v), src_tokens,
        src_tok0, reinterpret_cast<uint4*>(dst_k), reinterpret_cast<uint4*>(dst_v), dst_tokens,
        dst_tok0, n, row_vec, bh0, total);
    return hipGetLastError();
}

hipError_t launch_copy_one_ragged(const Layout& L, const DevPtrs& P, const void* src_k, const void* src_v,
                                  Ragged rg, hipStream_t stream) {
    const int row_vec = L.D * L.esize / 16;
    const int64_t total = L.BH * row_vec;
    const int grid = grid_for(2 * total, 256, 65535);
    copy_one_ragged_kernel<<<grid, 256, 0, stream>>>(
        reinterpret_cast<const uint4*>(src_k), reinterpret_cast<const uint4*>(src_v),
        reinterpret_cast<uint4*>(P.ksink), reinterpret_cast<uint4*>(P.vsink), reinterpret_cast<uint4*>(P.kres),
        reinterpret_cast<uint4*>(P.vres), rg.base_len, rg.delta, L.Hkv, L.S, L.R, L.Qf, row_vec, total);
    return hipGetLastError();
}

hipError_t launch_set_lengths(const Layout& L, int* base_len, const int64_t* lens, hipStream_t stream) {
    for (int b0 = 0; b0 < L.B; b0 += kLenChunk) {
        LenChunk c;
        c.n = std::min(kLenChunk, L.B - b0);
        for (int i = 0; i < c.n; ++i) c.v[i] = (int)lens[b0 + i];
        set_lengths_kernel<<<1, kLenChunk, 0, stream>>>(base_len + b0, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_set_entries(int* dst, const int* idx, const int* val, int n, hipStream_t stream) {
    for (int i0 = 0; i0 < n; i0 += kEntryChunk) {
        EntryChunk c;
        c.n = std::min(kEntryChunk, n - i0);
        for (int i = 0; i < c.n; ++i) c.idx[i] = idx[i0 + i], c.val[i] = val[i0 + i];
        set_entries_kernel<<<1, kEntryChunk, 0, stream>>>(dst, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_quantize(const Layout& L, const DevPtrs& P, const void* src_k, const void* src_v,
                           int64_t src_tokens, int64_t src_tok0, int64_t n_groups, int64_t dst_tok0,
                           int64_t bh0, int64_t nbh, hipStream_t stream, int tok_stride) {
    if (n_groups <= 0 || nbh <= 0) return hipSuccess;
    QuantArgs a;
    a.src_k = src_k;
    a.src_v = src_v;
    a.src_tokens = src_tokens;
    a.src_tok0 = src_tok0;
    a.dst_tok0 = dst_tok0;
    a.tok_stride = tok_stride;
    a.D = L.D;
    a.G = L.G;
    a.GV = L.GV;
    a.nvg = L.nvg;
    a.row_bytes = L.row_bytes;
    a.ng_cap = L.ng_cap;
    a.rec_bytes = L.rec_bytes;
    a.rec_kcodes = L.rec_kcodes;
    a.rec_vcodes = L.rec_vcodes;
    a.rec_vmeta = L.rec_vmeta;
    a.codec = L.codec;
    a.key_axis = L.key_axis;
    a.bh0 = bh0;
    a.rm = rec_map(L, P);
    a.outliers = L.outliers;
    a.rec_kov = L.rec_kov;
    a.rec_koi = L.rec_koi;
    a.rec_vov = L.rec_vov;
    a.rec_voi = L.rec_voi;
    // codes [G][D] bytes, then the keys' partial minima/maxima [P][D][2] fp32
    const size_t lds = (((size_t)L.G * L.D + 15) & ~(size_t)15) + (size_t)(256 / (L.D / 2)) * L.D * 2 * sizeof(float);
    dim3 grid((unsigned)n_groups, (unsigned)nbh);
#define KVQ_QLAUNCH(DT, BITS) quantize_kernel<DT, BITS><<<grid, 256, lds, stream>>>(a)
    if (L.bits == 4) {
        if (L.dtype == DT_F32) KVQ_QLAUNCH(DT_F32, 4);
        else if (L.dtype == DT_BF16) KVQ_QLAUNCH(DT_BF16, 4);
        else KVQ_QLAUNCH(DT_F16, 4);
    } else if (L.bits == 2) {
        if (L.dtype == DT_F32) KVQ_QLAUNCH(DT_F32, 2);
        else if (L.dtype == DT_BF16) KVQ_QLAUNCH(DT_BF16, 2);
        else KVQ_QLAUNCH(DT_F16, 2);
    } else {
        if (L.dtype == DT_F32) KVQ_QLAUNCH(DT_F32, 8);
        else if (L.dtype == DT_BF16) KVQ_QLAUNCH(DT_BF16, 8);
        else KVQ_QLAUNCH(DT_F16, 8);
    }
#undef KVQ_QLAUNCH
    return hipGetLastError();
}

hipError_t launch_flush(const Layout& L, const DevPtrs& P, int64_t Lq, int64_t bh0, int64_t nbh, hipStream_t stream) {
    if (L.Qf == L.R)
        return launch_quantize(L, P, P.kres, P.vres, L.R, 0, L.R / L.G, Lq, bh0, nbh, stream, 1);
    const int W = L.Qf;
    hipError_t e = launch_quantize(L, P, P.kres, P.vres, L.R, 0, W / L.G, Lq, bh0, nbh, stream, 2);
    if (e != hipSuccess || nbh <= 0) return e;
    const int row_vec = L.D * L.esize / 16;
    const int64_t total = nbh * row_vec;
    const int grid = grid_for(2 * total, 256, 65535);
    log_compact_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<uint4*>(P.kres), reinterpret_cast<uint4*>(P.vres),
                                                 L.R, W, row_vec, bh0, total);
    return hipGetLastError();
}

hipError_t launch_dequantize(const Layout& L, const DevPtrs& P, int64_t nS, int64_t Lq, int64_t r,
                             float* k_out, float* v_out, Ragged rg, hipStream_t stream) {
    DeqArgs a = make_deq_args(L, P, nS, Lq, r, rg);
    a.kout = k_out;
    a.vout = v_out;
    if (a.T == 0) return hipSuccess;
    dim3 grid(grid_for(a.T * L.D, 256, 4096), (unsigned)L.BH);
    if (L.dtype == DT_F32) dequantize_kernel<DT_F32><<<grid, 256, 0, stream>>>(a);
    else if (L.dtype == DT_BF16) dequantize_kernel<DT_BF16><<<grid, 256, 0, stream>>>(a);
    else dequantize_kernel<DT_F16><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_export(const Layout& L, const DevPtrs& P, int64_t Lq, uint8_t* k_codes,
                         float* k_scale, float* k_zero, uint8_t* v_codes, float* v_scale,
                         float* v_zero, Ragged rg, hipStream_t stream) {
    if (Lq == 0) return hipSuccess;
    DeqArgs a = make_deq_args(L, P, 0, Lq, 0, rg);
    dim3 grid(grid_for(Lq * L.D, 256, 4096), (unsigned)L.BH);
    export_kernel<<<grid, 256, 0, stream>>>(a, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero);
    return hipGetLastError();
}

hipError_t launch_export_outliers(const Layout& L, const DevPtrs& P, int64_t Lq, uint8_t* k_idx, float* k_val,
                                  uint8_t* v_idx, float* v_val, Ragged rg, hipStream_t stream) {
    if (Lq == 0) return hipSuccess;
    DeqArgs a = make_deq_args(L, P, 0, Lq, 0, rg);
    dim3 grid(grid_for(Lq * L.nvg, 256, 4096), (unsigned)L.BH);
    export_outliers_kernel<<<grid, 256, 0, stream>>>(a, k_idx, k_val, v_idx, v_val);
    return hipGetLastError();
}

}  // namespace kvq
