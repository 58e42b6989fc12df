// kvq_internal.h -- cache layout, packing format and kernel launch interfaces
// shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

constexpr int kWaves = 4;              // waves per decode / quantize workgroup
constexpr int kThreads = 64 * kWaves;  // 256 threads
constexpr int kMaxCombine = 1024;      // max (splits x query heads per kv head)
// Partials one workgroup merges in the split combine.  Up to kMaxMerge splits per
// slice merge in one level; more form groups of ceil(sqrt(nsplit)) splits, whose
// group partials merge in a second level, so a slice holds at most kMaxMerge^2.
constexpr int kMaxMerge = 16;
constexpr int kMaxSplits = kMaxMerge * kMaxMerge;

// ---------------------------------------------------------------------------
// Device buffer layout of one cache.  Slices bh = b * Hkv + kvh come first:
//   k_sink, v_sink : [BH][S][D]        storage dtype
//   k_res,  v_res  : [BH][R][D]        storage dtype
//   records        : [BH][Lq_cap / G]  one record of rec_bytes per key group
// Lq_cap = R * floor((max_tokens - S) / R): the largest quantized length a
// sequence of max_tokens tokens can reach.  A key group's record holds, in the
// order decode attention streams them:
//   kmeta  : fp32 [2][D]              key scales, then key zero points; with
//                                     per-token keys fp32 [G][2], (scale, zero)
//                                     of each token
//   kcodes : [G][D*bits/8]            key codes, one packed row per token
//   vcodes : [G/TB][D] uint32         value codes: for each block of TB = 32/bits
//                                     tokens, one dword per channel holding the
//                                     block's tokens (token j at pack_shift(bits, j))
//   vmeta  : fp32 [G][D/G_V][2]       value (scale, zero) per token and group
// so a slice's quantized tokens are one contiguous stream of records.  A packed
// field holds the code XOR code_bias(bits): for 4-bit codes the field is the
// two's-complement nibble of code - 8, which the decode kernel's signed 4-bit
// dot products take as is; for 8-bit codes it is the int8 code - 128, which the
// matrix cores' int8 products take as is.
// ---------------------------------------------------------------------------
struct Layout {
    int B, Hkv, Hq, D, bits, codec, G, GV, R, S, dtype, esize, gqa, nvg, row_bytes;
    int retention;  // kvq_retention
    int key_axis;   // kvq_key_axis: 0 keys per channel over G tokens, 1 per token over D channels
    int Qf;         // tokens quantized per flush: R, or W = R / 3 under log-sparse retention
    // Dense-and-sparse records (outliers = 1): after the value metadata, the key
    // outliers' exact values fp32 [D] and (token | code << 8) u16 [D], then the
    // value outliers' values fp32 [G][nvg] and (channel | code << 8) u16 [G][nvg].
    int outliers, rec_kov, rec_koi, rec_vov, rec_voi;
    int64_t BH, max_tokens, Lq_cap, ng_cap;
    int rec_bytes, rec_kcodes, rec_vcodes, rec_vmeta;
    // Paged records: P = 2^lp key groups of one sequence per page, all kv heads
    // ([Hkv][P] records, page_bytes), pages from a pool of pool_pages, located
    // through the table int32 [B][max_pages].  lp = -1: one contiguous stream of
    // ng_cap records per slice.
    int lp;
    int64_t pool_pages, max_pages, page_bytes;
    size_t off_ksink, off_vsink, off_kres, off_vres, off_rec, off_lens, off_table, total;
};

// Where the records of a cache are, for kernels: rec is the contiguous records
// ([BH][ng_cap] of rec_bytes) or the page pool; table (null when contiguous)
// maps (sequence, page) to a pool page.
struct RecMap {
    uint8_t* rec;
    const int* table;
    int64_t ng_cap, page_bytes;
    int rec_bytes, lp, max_pages, Hkv;
};

// Address of the record of key group grp of slice bh.
__host__ __device__ inline uint8_t* rec_ptr(const RecMap& m, int64_t bh, int64_t grp) {
    if (m.table == nullptr) return m.rec + (size_t)(bh * m.ng_cap + grp) * (size_t)m.rec_bytes;
    const int64_t b = bh / m.Hkv, kvh = bh % m.Hkv;
    const int64_t page = m.table[b * m.max_pages + (grp >> m.lp)];
    const int64_t in_page = kvh * ((int64_t)1 << m.lp) + (grp & (((int64_t)1 << m.lp) - 1));
    return m.rec + (size_t)(page * m.page_bytes) + (size_t)(in_page * m.rec_bytes);
}

// Sequences of different lengths.  Sequence b holds base_len[b] + delta tokens;
// base_len (int32 [B]) lives in the cache buffer, written by launch_set_lengths,
// and delta counts the one-token appends to every sequence since then.  A null
// base_len means every sequence has the length the launch is given.
struct Ragged {
    const int* base_len = nullptr;
    int delta = 0;
};

// Sinks held, quantized tokens and residual tokens of a sequence of n tokens:
// the first S tokens are sinks; the residual flushes when it holds R tokens,
// quantizing Q of them and keeping R - Q.  Whole-residual flushes (Q = R)
// quantize every run of R tokens; log-sparse retention (Q = R / 3) quantizes Q
// tokens once R are held and Q more after every further Q tokens.
struct SliceState {
    int nS, Lq, r;
};
__host__ __device__ inline SliceState slice_state(int64_t n, int S, int R, int Q) {
    const int64_t nS = n < S ? n : S;
    const int64_t m = n - nS;
    const int64_t Lq = m < R ? 0 : ((m - R) / Q + 1) * Q;
    return {(int)nS, (int)Lq, (int)(m - Lq)};
}

struct DevPtrs {
    char* ksink;
    char* vsink;
    char* kres;
    char* vres;
    uint8_t* rec;
    int* table;  // page table (paged records), else null
};

inline RecMap rec_map(const Layout& L, const DevPtrs& P) {
    return RecMap{P.rec, P.table, L.ng_cap, L.page_bytes, L.rec_bytes, L.lp, (int)L.max_pages, L.Hkv};
}

// ---------------------------------------------------------------------------
// Packing.  A token row of D codes is stored as D*bits/32 dwords.  Dword i of
// the row holds the 32/bits channels c = (32/bits)*i + j, j = 0..32/bits-1, with
// channel j in byte (j & 3) at bit offset bits * (j >> 2) inside that byte.
// Hence (dword >> (bits * k)) & (0x0F0F0F0F or 0x03030303) yields the four
// channels 4k..4k+3 of the dword as the four bytes of a word, ready for the
// byte-to-float conversions, and the unpacked order is the channel order.
// ---------------------------------------------------------------------------
__host__ __device__ inline int pack_shift(int bits, int j) { return 8 * (j & 3) + bits * (j >> 2); }
__host__ __device__ inline uint32_t code_bias(int bits) { return bits == 4 ? 8u : bits == 8 ? 128u : 0u; }

// Record addressing.
__host__ __device__ inline size_t rec_offset(int64_t bh, int64_t grp, int64_t ng_cap, int rec_bytes) {
    return (size_t)(bh * ng_cap + grp) * (size_t)rec_bytes;
}

// ---------------------------------------------------------------------------
// storage dtype helpers
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline float f16_to_f32(uint16_t h) {
    _Float16 x;
    __builtin_memcpy(&x, &h, 2);
    return (float)x;
}

template <int DT>
__device__ inline float load_as_f32(const void* base, int64_t idx) {
    if constexpr (DT == DT_F32) {
        return reinterpret_cast<const float*>(base)[idx];
    } else if constexpr (DT == DT_BF16) {
        return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    } else {
        return f16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    }
}

// ---------------------------------------------------------------------------
// launch interfaces (defined in the .hip sources)
// ---------------------------------------------------------------------------

// Copy n tokens of slices [bh0, bh0 + nbh) of K and V from src_*[bh][src_tok0 + i][D]
// (src holds src_tokens tokens per slice) to dst_*[bh][dst_tok0 + i][D] (dst holds
// dst_tokens per slice), in one launch.  Storage dtype preserved.
hipError_t launch_copy_tokens(const Layout& L, const void* src_k, const void* src_v,
                              int64_t src_tokens, int64_t src_tok0, char* dst_k, char* dst_v,
                              int64_t dst_tokens, int64_t dst_tok0, int64_t n, int64_t bh0, int64_t nbh,
                              hipStream_t stream);

// Quantize n_groups key groups (n_groups * G tokens) of slices [bh0, bh0 + nbh),
// token t read from src_k/src_v[bh][src_tok0 + t * tok_stride][D] (src_tokens
// rows per slice), into quantized token positions dst_tok0 + t.
hipError_t launch_quantize(const Layout& L, const DevPtrs& P, const void* src_k, const void* src_v,
                           int64_t src_tokens, int64_t src_tok0, int64_t n_groups, int64_t dst_tok0,
                           int64_t bh0, int64_t nbh, hipStream_t stream, int tok_stride = 1);

// Flush the full residual (R tokens) of slices [bh0, bh0 + nbh) whose quantized
// part holds Lq tokens: quantize all R (Qf == R), or, under log-sparse retention,
// quantize rows 0, 2, ..., 2W - 2 (W = Qf) and compact the rest to rows
// 0 .. 2W - 1.  Leaves Lq + Qf quantized tokens and R - Qf residual tokens.
hipError_t launch_flush(const Layout& L, const DevPtrs& P, int64_t Lq, int64_t bh0, int64_t nbh,
                        hipStream_t stream);

// One token per sequence (src_*[bh][D]) into each slice's own sink slot or residual
// row, from the sequence's length before the append (rg).
hipError_t launch_copy_one_ragged(const Layout& L, const DevPtrs& P, const void* src_k, const void* src_v,
                                  Ragged rg, hipStream_t stream);

// dst[idx[i]] = val[i] for i < n (host arrays), in launches of up to 256 entries.
hipError_t launch_set_entries(int* dst, const int* idx, const int* val, int n, hipStream_t stream);

// base_len[b] = lens[b] for b < L.B (lens: host array).
hipError_t launch_set_lengths(const Layout& L, int* base_len, const int64_t* lens, hipStream_t stream);

struct DecodeRequest {
    int64_t Lq;            // quantized tokens per slice
    int64_t nS, r;         // sinks held, residual tokens held
    int64_t split_tokens;  // tokens per split override (0 = automatic)
    int num_cu;            // compute units of the device
    int nsplit_cap;        // splits per slice the workspace holds
    // Fused one-token append: the newest residual token (index r - 1) is read from
    // these [B*Hkv][D] inputs instead of the residual, and split 0 of each slice
    // writes it to residual row r - 1.  Null for a plain decode.
    const void* knew = nullptr;
    const void* vnew = nullptr;
    // If set, HIP events that take the decode kernel's own start and end times.
    hipEvent_t ev_start = nullptr;
    hipEvent_t ev_stop = nullptr;
    // Sequences of different lengths: each slice's state comes from its length;
    // Lq, nS, r above are then those of the longest sequence (split plan, grid).
    Ragged rg;
};

hipError_t launch_decode(const Layout& L, const DevPtrs& P, const DecodeRequest& rq, const void* q,
                         float* out, float* lse, void* ws, float sm_scale, hipStream_t stream);

// true if an instantiation of the decode kernel serves this layout
bool decode_supported(const Layout& L);

size_t decode_workspace_bytes(const Layout& L, int max_splits);

// Static scratch for callers that cannot allocate: one file-scope device array of
// kStaticScratchBytes per device, laid out as a decode workspace.  Its device
// address (hipGetSymbolAddress, taken once per device with that device current)
// is returned in *ptr; the first call on a device also enqueues, on `stream`, a
// clear of the array (the completion counters must start at zero; every decode
// leaves them at zero).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(hipStream_t stream, void** ptr);

// Dequantize to [BH][T_out][D] fp32 (T_out = nS + Lq + r, the longest sequence's
// length with rg); with rg, rows past a slice's own length are not written.
hipError_t launch_dequantize(const Layout& L, const DevPtrs& P, int64_t nS, int64_t Lq, int64_t r,
                             float* k_out, float* v_out, Ragged rg, hipStream_t stream);

// Export codes [BH][Lq][D] and metadata (Lq of the longest sequence with rg; rows past
// a slice's own quantized length are not written).
hipError_t launch_export(const Layout& L, const DevPtrs& P, int64_t Lq, uint8_t* k_codes,
                         float* k_scale, float* k_zero, uint8_t* v_codes, float* v_scale,
                         float* v_zero, Ragged rg, hipStream_t stream);

// Export the outliers of dense-and-sparse records (layouts as kvq_export_outliers).
hipError_t launch_export_outliers(const Layout& L, const DevPtrs& P, int64_t Lq, uint8_t* k_idx, float* k_val,
                                  uint8_t* v_idx, float* v_val, Ragged rg, hipStream_t stream);

}  // namespace kvq
