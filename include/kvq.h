/*
 * kvq.h -- decode attention over a low-bit (INT2 / INT4 / INT8) KV cache on MI355X.
 *
 * The cache follows the KIVI scheme ("LLM系列：KVCache量化1 KIVI: A Tuning-Free
 * Asymmetric 2bit Quantiz", section 1 "KIVI"):
 *   - keys are quantized per channel, one group per G consecutive tokens;
 *   - values are quantized per token, one group per G_V consecutive channels;
 *   - the newest tokens sit in a full-precision residual of capacity R; when it
 *     holds R tokens they are quantized, appended to the quantized part, and the
 *     residual is emptied (or, under LogQuant's log-sparse retention, a thinned
 *     half of its oldest two thirds is quantized: see kvq_retention);
 *   - optionally the first S tokens of every sequence stay full precision for
 *     good ("attention sinks", "KV Cache的Int4量化：如何解决Attention Sink导致的量化精度
 *     崩塌问题", section 3).
 * Each group is quantized with asymmetric min-max parameters ("Atom: Low-bit
 * Quantization for Efficient and Accurate LLM Serving", section 三 "核心公式"):
 *   scale s = (max - min) / (2^n - 1)       zero z = round(-min / s)
 *   code  q = clamp(round(x / s) + z, 0, 2^n - 1)
 *   x'      = (q - z) * s                   (Int4 KV-cache post, section 2)
 * all in IEEE binary32, round half to even, in exactly that operation order.
 * A group whose scale comes out 0 (all values equal, or a range so small that
 * range / (2^n - 1) underflows) uses s = |min| (s = 1 when min == 0), so that it
 * reproduces exactly; a zero point of -0 is stored as +0.
 *
 * Decode attention computes, for every query head h of every sequence b,
 *   out = softmax(q K'^T * sm_scale) V'      (Int4 KV-cache post, section 3)
 * over all cached tokens of kv head h / (n_q_heads / n_kv_heads): the sinks, the
 * dequantized tokens and the residual (KIVI notes, section 1: logits of the
 * grouped and residual parts are concatenated before the softmax; the order of
 * tokens does not change the result, "Resumo Técnico: LogQuant", Metodologia 4).
 *
 * Conventions shared by every call:
 *   - All device memory (cache buffer, inputs, outputs, workspace) is owned by
 *     the caller and must stay alive until the enqueued work has finished.  The
 *     library owns only the host-side handle.  It never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call validates its arguments on the host before anything is
 *     enqueued; on error nothing is enqueued and the cache state is unchanged.
 *     Work is asynchronous on `stream`; the host never waits for the device.
 *   - Non-finite inputs, and inputs whose per-group range overflows binary32,
 *     give undefined (but memory-safe) results.
 *   - A handle is not thread-safe; calls on one handle must be serialized, and
 *     all of its work must be enqueued on streams ordered with each other.
 *   - kvq_last_error() returns a thread-local, library-owned message describing
 *     the last failed call on the calling thread.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,      /* bad pointer, shape or config value          */
    KVQ_ERR_UNSUPPORTED = -2,      /* valid but not supported by these kernels    */
    KVQ_ERR_CAPACITY = -3,         /* append would exceed max_tokens              */
    KVQ_ERR_BUFFER_TOO_SMALL = -4, /* cache buffer or workspace below the minimum */
    KVQ_ERR_DEVICE = -5            /* a HIP runtime or launch error               */
} kvq_status;

typedef enum kvq_dtype {
    KVQ_F32 = 0,
    KVQ_BF16 = 1,
    KVQ_F16 = 2
} kvq_dtype;

/*
 * Group quantizer of the cache ("Atom: Low-bit Quantization for Efficient and
 * Accurate LLM Serving", section 三 "核心公式"; clip factor 1):
 *   ASYMMETRIC: s = (max - min) / (2^n - 1), z = round(-min / s),
 *               code = clamp(round(x / s) + z, 0, 2^n - 1)
 *   SYMMETRIC:  s = 2 max|x| / (2^n - 1), signed code
 *               clamp(round(x / s), -2^(n-1), 2^(n-1) - 1), stored as that code
 *               + 2^(n-1), i.e. with z = 2^(n-1)
 * Both dequantize as x' = (code - z) s.  A group whose scale computes to 0 uses
 * |min| (asymmetric) or max|x| (symmetric), or 1 when that is 0.
 */
typedef enum kvq_codec {
    KVQ_CODEC_ASYMMETRIC = 0,
    KVQ_CODEC_SYMMETRIC = 1
} kvq_codec;

/*
 * Which tokens a flush quantizes when the full-precision residual reaches R
 * tokens:
 *   WINDOW: all R, leaving the residual empty (KIVI notes, "LLM系列：KVCache量化1
 *           KIVI…", section 1).
 *   LOG:    log-sparse retention ("Resumo Técnico: LogQuant", Metodologia
 *           item 2) with R = 3W, W a multiple of k_group: of the oldest 2W
 *           residual tokens, taken in pairs, the earlier of each pair is
 *           quantized (W tokens, W / G key groups, in their order) and the later
 *           kept; the kept W and the newest W remain, so 2W <= r < 3W after the
 *           first flush.  The kept tokens thin out with their distance from the
 *           newest token.  Attention does not depend on where a token is stored
 *           (same page, item 4), so quantized and kept tokens are stored in the
 *           order they were quantized or kept, not by position.
 */
typedef enum kvq_retention {
    KVQ_RETAIN_WINDOW = 0,
    KVQ_RETAIN_LOG = 1
} kvq_retention;

/*
 * Grouping of the keys:
 *   PER_CHANNEL: one group per channel over each run of G tokens (KIVI notes,
 *                "LLM系列：KVCache量化1 KIVI…", section 1: keys per channel).
 *   PER_TOKEN:   one group per token over its head_dim channels, i.e. one
 *                scale and zero point per token and kv head ("Atom: Low-bit
 *                Quantization for Efficient and Accurate LLM Serving", section
 *                三, model-components table, KV-cache row: asymmetric low-bit
 *                quantization at attention-head granularity).  G then only sets
 *                how many tokens a record holds: 64 or 128.  Not combined with
 *                outliers; with several query heads per kv head, or 8-bit codes,
 *                it needs G_V >= 64.
 */
typedef enum kvq_key_axis {
    KVQ_KEY_PER_CHANNEL = 0,
    KVQ_KEY_PER_TOKEN = 1
} kvq_key_axis;

typedef struct kvq_config {
    int32_t batch;        /* B  >= 1                                              */
    int32_t n_kv_heads;   /* Hkv >= 1                                             */
    int32_t n_q_heads;    /* Hq, a multiple of Hkv; Hq / Hkv in {1, 2, 4, 8}      */
    int32_t head_dim;     /* D in {64, 128}                                       */
    int32_t bits;         /* n in {2, 4, 8}; 8-bit codes need G >= 64 and G_V   */
                          /* >= 64.  Mixed precision per layer: one cache per    */
                          /* layer, each with its own bits                       */
    int32_t k_group;      /* G: tokens per key group; 32, 64, 128 or 256          */
    int32_t v_group;      /* G_V: channels per value group; divides D, a multiple */
                          /* of 16                                                */
    int32_t residual;     /* R: residual capacity; a multiple of G                */
    int32_t n_sink;       /* S >= 0: leading tokens kept at full precision        */
    int32_t dtype;        /* kvq_dtype of K, V, q and of the sink/residual store  */
    int64_t max_tokens;   /* capacity per sequence, >= 1                          */
    float sm_scale;       /* softmax scale; 0 selects 1/sqrt(D)                   */
    int32_t codec;        /* kvq_codec of the key and value groups (0: asymmetric) */
    int32_t retention;    /* kvq_retention of the residual flush (0: window)      */
    int32_t page_groups;  /* P: key groups per page of paged records, a power of  */
                          /* two; 0 stores each sequence's records contiguously  */
    int64_t pool_pages;   /* pages in the pool (paged records); 0 = enough for    */
                          /* every sequence at max_tokens                         */
    int32_t outliers;     /* 1: one full-precision outlier per quantization vector */
                          /* (dense-and-sparse groups, see kvq_export_outliers)   */
    int32_t key_axis;     /* kvq_key_axis of the key groups (0: per channel)      */
} kvq_config;

typedef struct kvq_cache kvq_cache; /* opaque host-side handle */

/*
 * Minimum size in bytes of the device buffer that holds a cache of `cfg`:
 * sinks, residual, packed codes and scales/zero points for max_tokens tokens
 * per sequence.  Errors: INVALID_ARG / UNSUPPORTED as for kvq_cache_create.
 */
kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes);

/*
 * Create an empty cache in the caller's device buffer `dev_buf` (>= the size
 * from kvq_cache_bytes, 256-byte aligned).  The buffer's contents need no
 * initialisation.  *out receives the handle, to be freed with
 * kvq_cache_destroy.  Errors: INVALID_ARG (null pointer, non-positive sizes,
 * Hq % Hkv != 0, R % G != 0, D % G_V != 0, codec not a kvq_codec, retention not a
 * kvq_retention, key_axis not a kvq_key_axis, log-sparse retention with R not a
 * multiple of 3G, page_groups not 0 or a power of two, pool_pages < 0, misaligned
 * buffer),
 * UNSUPPORTED (bits not 2/4/8, D not 64/128, Hq/Hkv not 1/2/4/8, G not in
 * {32, 64, 128, 256}, G_V not a multiple of 16, 8-bit codes with G or G_V
 * below 64, per-token keys with G not 64 or 128, with outliers, or with G_V
 * below 64 where several query heads share a kv head or codes are 8-bit,
 * B * Hkv > 65535, more than
 * 2 GiB of quantized records per (sequence, kv head), a page pool above 4 GiB,
 * pages so small that a decode split would span more than 63 of them), BUFFER_TOO_SMALL,
 * DEVICE (no current HIP device).
 */
kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes,
                            kvq_cache** out);

/* Free a handle (NULL is accepted).  The device buffer stays the caller's. */
kvq_status kvq_cache_destroy(kvq_cache* cache);

/*
 * Append n_new tokens to every sequence (KIVI notes, section 1: the new key
 * and value go to the residual; the residual is quantized and appended to the
 * grouped part when it reaches R tokens).  Equivalent, bit for bit, to n_new
 * one-token appends: the first S tokens ever appended become sinks, each later
 * token goes to residual slot r, and whenever r reaches R the R residual
 * tokens are quantized (keys per channel over each run of G tokens, values per
 * token over each run of G_V channels) and the residual is emptied, so that
 * 0 <= r < R after every call.  Complete R-token blocks of a bulk append are
 * quantized straight from the input.  Under log-sparse retention a flush
 * quantizes W of the R tokens instead and keeps 2W (kvq_retention), and a bulk
 * append passes through the residual.  Each sequence follows this from its own
 * length when the sequences differ in length (see kvq_append_ragged).
 *   k, v : device, [B, Hkv, n_new, D] contiguous, in cfg.dtype.
 * n_new == 0 is a no-op.  Errors: INVALID_ARG (null, n_new < 0),
 * CAPACITY (the longest sequence's tokens + n_new > max_tokens), DEVICE.
 */
kvq_status kvq_append(kvq_cache* cache, const void* k, const void* v, int64_t n_new,
                      void* stream);

/*
 * Size in bytes of the decode workspace for this cache (split partials and
 * completion counters; constant over the cache's lifetime).
 */
kvq_status kvq_decode_workspace_bytes(const kvq_cache* cache, size_t* bytes);

/*
 * Decode attention for one query per (sequence, query head):
 *   out[b, h, :] = softmax(q[b, h] . K'^T * sm_scale) V'
 *   lse[b, h]    = log(sum(exp(q[b, h] . K'^T * sm_scale)))   (natural log)
 * over every cached token of kv head h / (Hq / Hkv) (of sequence b's own
 * length when the sequences differ in length).  The keys and values of
 * the quantized part are dequantized on the fly; the token range is split
 * across workgroups and the partial softmax states are merged with a
 * log-sum-exp combine.
 *   q   : device, [B, Hq, D] in cfg.dtype.
 *   out : device, [B, Hq, D] fp32.       lse : device, [B, Hq] fp32, or NULL.
 *   ws  : device workspace of >= kvq_decode_workspace_bytes bytes, 256-byte
 *         aligned, ZERO-FILLED before its first use; every call leaves its
 *         counters zero again.  Calls that share a workspace must not overlap.
 * The result matches the binary64 definition to within about 1e-4 absolute for
 * the documented workloads.  Errors: INVALID_ARG (null q/out/ws, an empty
 * sequence), BUFFER_TOO_SMALL (ws), DEVICE.
 */
kvq_status kvq_decode_attention(kvq_cache* cache, const void* q, float* out, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * kvq_decode_attention for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation and result, bit for bit, with the
 * workspace taken from a static array inside the library instead of `ws`.
 *   - The array holds 16 MiB per device (KVQ_STATIC_SCRATCH_BYTES) and is
 *     allocated when the library is loaded; each device the library runs on
 *     keeps its own copy until the process ends.  The call itself allocates
 *     nothing.
 *   - Every call on one device shares that device's array: calls that overlap
 *     on one device (on different streams or threads) race and give undefined
 *     results.  Calls ordered on one stream are safe.
 *   - The first call on a device clears the array on `stream` before its decode;
 *     every call leaves the array's completion counters at zero for the next.
 *   q, out, lse, stream : as for kvq_decode_attention.
 * Errors: those of kvq_decode_attention, and BUFFER_TOO_SMALL when this cache's
 * decode needs more than KVQ_STATIC_SCRATCH_BYTES of workspace
 * (kvq_decode_workspace_bytes), checked before anything is enqueued.
 */
#define KVQ_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
kvq_status kvq_decode_attention_static(kvq_cache* cache, const void* q, float* out, float* lse, void* stream);

/*
 * One decode step in one call: append one token per sequence, then decode
 * attention with the given query; the result and the cache state are exactly
 * those of kvq_append(cache, k, v, 1, stream) followed by
 * kvq_decode_attention(cache, q, out, lse, ws, ws_bytes, stream) (KIVI notes,
 * section 1: the step's key and value join the residual before the logits of
 * the grouped part and the residual are concatenated).  When every sequence's
 * token goes to its residual without filling it, the append happens inside the
 * decode launch (the kernel reads the new tokens from k and v and stores each
 * into its sequence's residual row, sequences of different lengths included);
 * when some token becomes a sink or fills its residual (a flush), the step takes
 * the two-call path.
 *   k, v : device, [B, Hkv, 1, D] contiguous, in cfg.dtype, 16-byte aligned;
 *          they must stay unmodified until the enqueued work completes.
 *   q, out, lse, ws : as for kvq_decode_attention.
 * Errors: those of kvq_append and kvq_decode_attention; nothing is enqueued and
 * the state is unchanged when validation fails.
 */
kvq_status kvq_append_decode(kvq_cache* cache, const void* k, const void* v, const void* q,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantize the whole cache to fp32 in storage order (sinks, then the quantized
 * tokens as x' = (q - z) * s in the order they were quantized, then the
 * residual; chronological order under window retention); the round trip
 * of the Int4 KV-cache post's section 5.1 `quantize` helper.
 *   k_out, v_out : device, [B, Hkv, n_tokens, D] fp32 (n_tokens of
 *                  kvq_cache_state; rows past a shorter sequence's own length
 *                  are not written).
 * Errors: INVALID_ARG (null), DEVICE.
 */
kvq_status kvq_dequantize(const kvq_cache* cache, float* k_out, float* v_out, void* stream);

/*
 * Export the quantized part in a canonical, unpacked layout (for bit-exact
 * comparison; independent of the internal packing):
 *   k_codes, v_codes : device uint8 [B, Hkv, n_quant, D]
 *   k_scale, k_zero  : device fp32  [B, Hkv, n_quant / G, D]; with
 *                      KVQ_KEY_PER_TOKEN keys [B, Hkv, n_quant, 1]
 *   v_scale, v_zero  : device fp32  [B, Hkv, n_quant, D / G_V]
 * (n_quant of kvq_cache_state; rows past a shorter sequence's own quantized
 * tokens are not written).  Any pointer may be NULL to skip that array.
 * Errors: DEVICE.
 */
kvq_status kvq_export(const kvq_cache* cache, uint8_t* k_codes, float* k_scale, float* k_zero,
                      uint8_t* v_codes, float* v_scale, float* v_zero, void* stream);

/*
 * Host-side counters (no device access): total tokens per sequence, sinks
 * held, quantized tokens and residual tokens.  When the sequences differ in
 * length: those of the longest sequence.  Any pointer may be NULL.
 */
kvq_status kvq_cache_state(const kvq_cache* cache, int64_t* n_tokens, int64_t* n_sink,
                           int64_t* n_quant, int64_t* n_resid);

/*
 * Append a different number of tokens to each sequence: sequence b takes the
 * first n_new[b] of its rows, as n_new[b] one-token appends from its own state
 * (sinks, residual and flushes exactly as for kvq_append; KIVI notes,
 * section 1).  The sequences then differ in length: every later call follows
 * each sequence's own length (kvq_append of one token per sequence writes each
 * token to its own slot and flushes only the sequences whose residual fills;
 * decode attention, dequantize and export use each slice's own tokens).  The
 * cache returns to the uniform layout's fast paths when the lengths agree again.
 *   k, v  : device, [B, Hkv, n_max, D] contiguous, in cfg.dtype (rows past
 *           n_new[b] are not read).
 *   n_new : host, int32 [B], each in [0, n_max].
 * All zero is a no-op.  Validation is complete before anything is enqueued.
 * The sequence lengths live in the cache buffer, written on `stream`.
 * Errors: INVALID_ARG (null, n_max < 0, n_new[b] outside [0, n_max]),
 * CAPACITY (a sequence would exceed max_tokens, or the page pool has too few
 * free pages), DEVICE.
 */
kvq_status kvq_append_ragged(kvq_cache* cache, const void* k, const void* v, const int32_t* n_new,
                             int64_t n_max, void* stream);

/*
 * Host-side: tokens held by each sequence, lens[b] for b < B (host array).
 * Errors: INVALID_ARG (null).
 */
kvq_status kvq_seq_lengths(const kvq_cache* cache, int64_t* lens);

/*
 * Paged records (cfg.page_groups = P > 0), as a page table manages a serving
 * KV cache ("Atom: Low-bit Quantization for Efficient and Accurate LLM
 * Serving", runtime-breakdown figure: self-attention through PageAttention, and
 * the baselines' list: vLLM keeps the KV cache under a page table to use GPU
 * memory fully).  The quantized records of a sequence live in pages of P key
 * groups (all kv heads of those groups), taken from a pool of cfg.pool_pages
 * pages in the cache buffer as the sequence's quantized part grows and located
 * through a page table [B][ceil(Lq_cap / (G P))] in the cache buffer.  Sinks and
 * the residual stay per sequence.  Results are bitwise those of contiguous
 * records.  An append that needs more pages than the pool has free fails with
 * CAPACITY and changes nothing.  The pool is at most 4 GiB.
 *
 * Release sequence b: its pages return to the pool and it becomes empty (length
 * 0), ready to take a new sequence; the other sequences are unchanged.  Work
 * already enqueued on `stream` that reads the released pages completes before
 * later appends on the same stream reuse them.  Also valid for contiguous records
 * (the sequence is emptied).  Decode attention needs every sequence non-empty.
 * Errors: INVALID_ARG (null, b outside [0, B)), DEVICE.
 */
kvq_status kvq_release_sequence(kvq_cache* cache, int32_t b, void* stream);

/*
 * Dense-and-sparse groups (cfg.outliers = 1; "LLM系列：KVCache量化1 KIVI…" page,
 * section 3 "KVQuant", item (4): per-vector dense-and-sparse quantization keeps
 * a small share of numeric outliers, e.g. 1%, unquantized in a sparse matrix).
 * Every quantization vector (a key channel over a group of G tokens, a token's
 * G_V value channels) has one outlier: its element of largest magnitude, the
 * lowest index among equal magnitudes.  The vector's scale and zero point come
 * from its other elements; every element still has a code (the outlier's
 * clamped like any other); the outlier dequantizes to its exact value, which is
 * what attention, kvq_dequantize and this export use.  kvq_export gives the
 * codes and metadata as without outliers.
 *   k_idx, k_val : device, [B, Hkv, n_quant / G, D] uint8 / fp32: the outlier's
 *                  token within each key group (per channel) and its value.
 *   v_idx, v_val : device, [B, Hkv, n_quant, D / G_V] uint8 / fp32: the outlier's
 *                  channel within each value group (per token) and its value.
 * Any output may be NULL (skipped).  Rows past a shorter sequence's own are not
 * written.  Errors: INVALID_ARG (null cache, a cache without outliers), DEVICE.
 * Decode attention with outliers runs for 2- and 4-bit codes (any number of
 * query heads per kv head); 8-bit codes with outliers are UNSUPPORTED at creation.
 */
kvq_status kvq_export_outliers(const kvq_cache* cache, uint8_t* k_idx, float* k_val, uint8_t* v_idx,
                               float* v_val, void* stream);

/* Host-side: free pages of the pool (0 for contiguous records).  Errors: INVALID_ARG. */
kvq_status kvq_pool_free_pages(const kvq_cache* cache, int64_t* free_pages);

/*
 * Tuning and testing knob: tokens per decode split of the quantized part
 * (rounded up to whole key groups).  0 restores the automatic choice.  The
 * result does not depend on the split, up to floating-point reassociation.
 * Errors: INVALID_ARG (negative).
 */
kvq_status kvq_set_split_tokens(kvq_cache* cache, int64_t tokens_per_split);

/*
 * Measurement hook: every later decode launch of this cache (kvq_decode_attention,
 * kvq_append_decode) records start_event at the start of its decode kernel and
 * stop_event at its end, so hipEventElapsedTime(start, stop) is the kernel's own
 * duration, without the dispatch gaps that events recorded around the call
 * include.  Both are hipEvent_t handles created by the caller with timing
 * enabled; the caller keeps them alive while a launch that records them is
 * pending.  NULL, NULL stops the recording.  A launch that takes two kernels
 * (an append that flushes, then the decode) records the decode kernel only.
 * Errors: INVALID_ARG (NULL cache, or exactly one event NULL).
 */
kvq_status kvq_set_timing_events(kvq_cache* cache, void* start_event, void* stop_event);

/*
 * Measurement hook, independent of any cache: one plain streaming read of
 * `bytes` of device memory at `buf` (16-byte loads, eight in flight per
 * thread, blocks_per_cu workgroups of 256 threads per compute unit of the
 * current device), enqueued on `stream`.  Timed by the caller, it gives the
 * read bandwidth that a kernel streaming its input once can reach on this
 * device.  The data is folded with XOR; `sink` (4 device bytes) is written
 * only when the fold equals one fixed word, so its contents are meaningless.
 * buf: 16-byte aligned, bytes a multiple of 16.  Nothing is allocated.
 * Errors: INVALID_ARG (NULL or misaligned pointers, blocks_per_cu outside
 * [1, 64]); DEVICE (launch failure).
 */
kvq_status kvq_stream_read_probe(const void* buf, size_t bytes, int32_t blocks_per_cu, uint32_t* sink,
                                 void* stream);

/* Message of the last failed call on this thread ("" if none).  Library-owned. */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
