// kvq_host.cpp -- the C-ABI of libkvq: config validation, the cache state
// machine (sinks / quantized groups / residual), split planning and kernel
// launches on the caller's stream.  The host never waits on the device.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

using namespace kvq;

static_assert(KVQ_STATIC_SCRATCH_BYTES == kStaticScratchBytes, "the header states the static scratch's size");

namespace kvq {
// probe.hip: one streaming read of n16 16-byte words at buf with `blocks` workgroups of 256
hipError_t launch_stream_read(const void* buf, int64_t n16, int blocks, unsigned* sink, hipStream_t stream);
}  // namespace kvq

struct kvq_cache {
    Layout L;
    DevPtrs P;
    char* buf;
    int64_t nS, Lq, r;        // sinks held, quantized tokens, residual tokens (all sequences
                              // alike; with `ragged`, those of the longest sequence)
    bool ragged = false;      // the sequences differ in length
    std::vector<int64_t> len; // tokens per sequence
    int len_delta = 0;        // one-token appends to every sequence since base_len was set
    int* base_len = nullptr;  // device int32 [B] in the cache buffer (ragged caches)
    int64_t split_tokens;     // 0 = automatic
    int num_cu;
    int nsplit_cap;           // max splits per slice the workspace holds
    float sm_scale;
    hipEvent_t ev_start = nullptr, ev_stop = nullptr;  // decode kernel timing (caller's events)
    // paged records: host copy of the page table ([B][max_pages], -1 = none), the
    // free pages (a stack) and the pages each sequence holds
    std::vector<int> table;
    std::vector<int> free_pages;
    std::vector<int> n_pages;
};

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kvq_status ok() {
    g_err[0] = '\0';
    return KVQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(const kvq_config* c);

kvq_status validate(const kvq_config* c) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "config is NULL");
    if (c->codec != KVQ_CODEC_ASYMMETRIC && c->codec != KVQ_CODEC_SYMMETRIC)
        return fail(KVQ_ERR_INVALID_ARG, "codec must be KVQ_CODEC_ASYMMETRIC or KVQ_CODEC_SYMMETRIC");
    if (c->retention != KVQ_RETAIN_WINDOW && c->retention != KVQ_RETAIN_LOG)
        return fail(KVQ_ERR_INVALID_ARG, "retention must be KVQ_RETAIN_WINDOW or KVQ_RETAIN_LOG");
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->head_dim < 1)
        return fail(KVQ_ERR_INVALID_ARG, "batch, heads and head_dim must be positive");
    if (c->n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                    c->n_q_heads, c->n_kv_heads);
    if (c->k_group < 1 || c->v_group < 1 || c->residual < 1)
        return fail(KVQ_ERR_INVALID_ARG, "k_group, v_group and residual must be positive");
    if (c->residual % c->k_group != 0)
        return fail(KVQ_ERR_INVALID_ARG, "residual (%d) is not a multiple of k_group (%d)",
                    c->residual, c->k_group);
    if (c->head_dim % c->v_group != 0)
        return fail(KVQ_ERR_INVALID_ARG, "head_dim (%d) is not a multiple of v_group (%d)",
                    c->head_dim, c->v_group);
    if (c->outliers != 0 && c->outliers != 1) return fail(KVQ_ERR_INVALID_ARG, "outliers must be 0 or 1");
    if (c->key_axis != KVQ_KEY_PER_CHANNEL && c->key_axis != KVQ_KEY_PER_TOKEN)
        return fail(KVQ_ERR_INVALID_ARG, "key_axis must be KVQ_KEY_PER_CHANNEL or KVQ_KEY_PER_TOKEN");
    if (c->page_groups < 0 || (c->page_groups & (c->page_groups - 1)) != 0)
        return fail(KVQ_ERR_INVALID_ARG, "page_groups (%d) must be 0 or a power of two", c->page_groups);
    if (c->pool_pages < 0) return fail(KVQ_ERR_INVALID_ARG, "pool_pages must be >= 0");
    if (c->retention == KVQ_RETAIN_LOG && c->residual % (3 * c->k_group) != 0)
        return fail(KVQ_ERR_INVALID_ARG, "log-sparse retention needs residual = 3W with W a multiple of "
                    "k_group (residual %d, k_group %d)", c->residual, c->k_group);
    if (c->n_sink < 0) return fail(KVQ_ERR_INVALID_ARG, "n_sink must be >= 0");
    if (c->max_tokens < 1) return fail(KVQ_ERR_INVALID_ARG, "max_tokens must be >= 1");
    if (c->dtype != KVQ_F32 && c->dtype != KVQ_BF16 && c->dtype != KVQ_F16)
        return fail(KVQ_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
    if (!(c->sm_scale >= 0.0f) || isinf(c->sm_scale))
        return fail(KVQ_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
    if (c->bits != 2 && c->bits != 4 && c->bits != 8) return fail(KVQ_ERR_UNSUPPORTED, "bits must be 2, 4 or 8");
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    const int g = c->n_q_heads / c->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(KVQ_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (c->k_group != 32 && c->k_group != 64 && c->k_group != 128 && c->k_group != 256)
        return fail(KVQ_ERR_UNSUPPORTED, "k_group must be 32, 64, 128 or 256");
    if (c->v_group < 16 || c->v_group % 16 != 0)
        return fail(KVQ_ERR_UNSUPPORTED, "v_group must be a multiple of 16");
    if ((int64_t)c->batch * c->n_kv_heads > 65535)
        return fail(KVQ_ERR_UNSUPPORTED, "batch * n_kv_heads must be at most 65535");
    if (c->key_axis == KVQ_KEY_PER_TOKEN) {
        if (c->k_group != 64 && c->k_group != 128)
            return fail(KVQ_ERR_UNSUPPORTED, "per-token keys need k_group 64 or 128");
        if (c->outliers) return fail(KVQ_ERR_UNSUPPORTED, "per-token keys do not take outliers");
    }
    {   // the decode kernel addresses one slice's records, or the page pool, with
        // 32-bit offsets
        const Layout L = make_layout(c);
        if (L.lp < 0 && L.ng_cap * (int64_t)L.rec_bytes > (int64_t)INT32_MAX)
            return fail(KVQ_ERR_UNSUPPORTED, "max_tokens %lld gives more than 2 GiB of quantized "
                        "records per (sequence, kv head)", (long long)c->max_tokens);
        if (L.lp >= 0 && L.pool_pages * L.page_bytes > (int64_t)UINT32_MAX)
            return fail(KVQ_ERR_UNSUPPORTED, "the page pool (%lld pages of %lld bytes) exceeds 4 GiB",
                        (long long)L.pool_pages, (long long)L.page_bytes);
    }
    return KVQ_OK;
}

Layout make_layout(const kvq_config* c) {
    Layout L;
    L.B = c->batch;
    L.Hkv = c->n_kv_heads;
    L.Hq = c->n_q_heads;
    L.D = c->head_dim;
    L.bits = c->bits;
    L.codec = c->codec;
    L.retention = c->retention;
    L.G = c->k_group;
    L.GV = c->v_group;
    L.R = c->residual;
    L.Qf = c->retention == KVQ_RETAIN_LOG ? c->residual / 3 : c->residual;
    L.S = c->n_sink;
    L.dtype = c->dtype;
    L.esize = c->dtype == KVQ_F32 ? 4 : 2;
    L.gqa = L.Hq / L.Hkv;
    L.nvg = L.D / L.GV;
    L.row_bytes = L.D * L.bits / 8;
    L.BH = (int64_t)L.B * L.Hkv;
    L.max_tokens = c->max_tokens;
    {   // the quantized tokens of a full sequence (slice_state, in 64-bit)
        const int64_t m = std::max<int64_t>(0, c->max_tokens - L.S);
        L.Lq_cap = m < L.R ? 0 : ((m - L.R) / L.Qf + 1) * L.Qf;
    }
    L.ng_cap = L.Lq_cap / L.G;
    L.key_axis = c->key_axis;
    L.rec_kcodes = 8 * (L.key_axis == KVQ_KEY_PER_TOKEN ? L.G : L.D);  // key (scale, zero): [2][D] or [G][2]
    L.rec_vcodes = L.rec_kcodes + L.G * L.row_bytes;
    L.rec_vmeta = L.rec_vcodes + L.G * L.row_bytes;
    L.outliers = c->outliers;
    L.rec_kov = L.rec_vmeta + L.G * L.nvg * 8;
    L.rec_koi = L.rec_kov + 4 * L.D;
    L.rec_vov = L.rec_koi + 2 * L.D;
    L.rec_voi = L.rec_vov + 4 * L.G * L.nvg;
    const int rec_end = L.outliers ? L.rec_voi + 2 * L.G * L.nvg : L.rec_kov;
    L.rec_bytes = (int)align256((size_t)rec_end);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t fp_row = (size_t)L.D * L.esize;
    L.off_ksink = take((size_t)L.BH * L.S * fp_row);
    L.off_vsink = take((size_t)L.BH * L.S * fp_row);
    L.off_kres = take((size_t)L.BH * L.R * fp_row);
    L.off_vres = take((size_t)L.BH * L.R * fp_row);
    if (c->page_groups > 0) {
        int lp = 0;
        while ((1 << lp) < c->page_groups) ++lp;
        L.lp = lp;
        L.max_pages = (L.ng_cap + c->page_groups - 1) / c->page_groups;
        L.page_bytes = (int64_t)L.Hkv * c->page_groups * L.rec_bytes;
        L.pool_pages = c->pool_pages > 0 ? c->pool_pages : (int64_t)L.B * L.max_pages;
        L.off_rec = take((size_t)(L.pool_pages * L.page_bytes));
    } else {
        L.lp = -1;
        L.max_pages = 0;
        L.page_bytes = 0;
        L.pool_pages = 0;
        L.off_rec = take((size_t)L.BH * L.ng_cap * L.rec_bytes);
    }
    L.off_lens = take((size_t)L.B * sizeof(int));
    L.off_table = take((size_t)L.B * L.max_pages * sizeof(int));
    L.total = off;
    return L;
}

kvq_status check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(KVQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return KVQ_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes) {
    kvq_status st = validate(cfg);
    if (st != KVQ_OK) return st;
    if (!bytes) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    const Layout L = make_layout(cfg);
    if (!decode_supported(L)) return fail(KVQ_ERR_UNSUPPORTED, "no decode kernel for this configuration");
    *bytes = L.total;
    return ok();
}

kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes, kvq_cache** out) {
    kvq_status st = validate(cfg);
    if (st != KVQ_OK) return st;
    if (!dev_buf || !out) return fail(KVQ_ERR_INVALID_ARG, "dev_buf or out is NULL");
    if (!aligned(dev_buf, 256)) return fail(KVQ_ERR_INVALID_ARG, "dev_buf must be 256-byte aligned");
    Layout L = make_layout(cfg);
    if (!decode_supported(L)) return fail(KVQ_ERR_UNSUPPORTED, "no decode kernel for this configuration");
    if (bytes < L.total)
        return fail(KVQ_ERR_BUFFER_TOO_SMALL, "cache buffer holds %zu bytes, needs %zu", bytes, L.total);
    int dev = 0, ncu = 0;
    if ((st = check_hip(hipGetDevice(&dev), "hipGetDevice")) != KVQ_OK) return st;
    if ((st = check_hip(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev),
                        "hipDeviceGetAttribute")) != KVQ_OK)
        return st;
    kvq_cache* c = new (std::nothrow) kvq_cache;
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "out of host memory");
    c->L = L;
    c->buf = (char*)dev_buf;
    c->P.ksink = c->buf + L.off_ksink;
    c->P.vsink = c->buf + L.off_vsink;
    c->P.kres = c->buf + L.off_kres;
    c->P.vres = c->buf + L.off_vres;
    c->P.rec = (uint8_t*)(c->buf + L.off_rec);
    c->P.table = L.lp >= 0 ? reinterpret_cast<int*>(c->buf + L.off_table) : nullptr;
    c->nS = c->Lq = c->r = 0;
    c->ragged = false;
    c->len.assign((size_t)L.B, 0);
    c->len_delta = 0;
    c->base_len = reinterpret_cast<int*>(c->buf + L.off_lens);
    c->split_tokens = 0;
    c->num_cu = ncu > 0 ? ncu : 256;
    const int64_t want = std::max<int64_t>(8, (16LL * c->num_cu + L.BH - 1) / L.BH);
    const int64_t cap_q = std::min<int64_t>(std::min<int64_t>(want, kMaxSplits - 1), kMaxCombine / L.gqa - 1);
    c->nsplit_cap = (int)cap_q + 1;
    if (L.lp >= 0) {
        // a decode split spans at most 63 pages' worth of key groups
        const int64_t per_split = 63 * ((int64_t)1 << L.lp);
        if ((L.ng_cap + per_split - 1) / per_split > cap_q) {
            delete c;
            return fail(KVQ_ERR_UNSUPPORTED, "page_groups %d is too small for max_tokens %lld: decode "
                        "splits would span more than 63 pages", 1 << L.lp, (long long)L.max_tokens);
        }
        c->table.assign((size_t)(L.B * L.max_pages), -1);
        c->free_pages.resize((size_t)L.pool_pages);
        for (int64_t i = 0; i < L.pool_pages; ++i) c->free_pages[(size_t)i] = (int)(L.pool_pages - 1 - i);
        c->n_pages.assign((size_t)L.B, 0);
    }
    c->sm_scale = cfg->sm_scale > 0.0f ? cfg->sm_scale : (float)(1.0 / sqrt((double)L.D));
    *out = c;
    return ok();
}

kvq_status kvq_cache_destroy(kvq_cache* cache) {
    delete cache;
    return ok();
}

}  // extern "C"

namespace {

// Appends n_new tokens (src_*[bh][src_tokens][D], tokens 0 .. n_new - 1) to slices
// [bh0, bh0 + nbh), which all hold the state st (updated).  Sinks first, then a
// partly filled residual (flushed when it reaches R), then whole R-token blocks
// quantized straight from the input, then the remainder as a new residual.
// Under log-sparse retention each flush keeps 2W residual tokens, so the input
// goes through the residual W tokens at a time.
kvq_status append_slices(kvq_cache* c, const void* k, const void* v, int64_t n_new, int64_t src_tokens,
                         int64_t bh0, int64_t nbh, SliceState& st, hipStream_t s) {
    const Layout& L = c->L;
    kvq_status e;
    int64_t src = 0, rem = n_new;
    // 1. sinks
    if (st.nS < L.S && rem > 0) {
        const int64_t take = std::min<int64_t>(L.S - st.nS, rem);
        if ((e = check_hip(launch_copy_tokens(L, k, v, src_tokens, src, c->P.ksink, c->P.vsink, L.S, st.nS,
                                              take, bh0, nbh, s),
                           "append")))
            return e;
        st.nS += (int)take;
        src += take;
        rem -= take;
    }
    if (L.Qf != L.R) {
        while (rem > 0) {
            const int64_t take = std::min<int64_t>(L.R - st.r, rem);
            if ((e = check_hip(launch_copy_tokens(L, k, v, src_tokens, src, c->P.kres, c->P.vres, L.R, st.r,
                                                  take, bh0, nbh, s),
                               "append")))
                return e;
            st.r += (int)take;
            src += take;
            rem -= take;
            if (st.r == L.R) {
                if ((e = check_hip(launch_flush(L, c->P, st.Lq, bh0, nbh, s), "flush"))) return e;
                st.Lq += L.Qf;
                st.r = L.R - L.Qf;
            }
        }
        return KVQ_OK;
    }
    // 2. top up a partly filled residual; flush it when it reaches R
    if (rem > 0 && st.r > 0) {
        const int64_t take = std::min<int64_t>(L.R - st.r, rem);
        if ((e = check_hip(launch_copy_tokens(L, k, v, src_tokens, src, c->P.kres, c->P.vres, L.R, st.r, take,
                                              bh0, nbh, s),
                           "append")))
            return e;
        st.r += (int)take;
        src += take;
        rem -= take;
        if (st.r == L.R) {
            if ((e = check_hip(launch_flush(L, c->P, st.Lq, bh0, nbh, s), "flush"))) return e;
            st.Lq += L.R;
            st.r = 0;
        }
    }
    // 3. complete R-token blocks straight from the input
    const int64_t nblk = rem / L.R;
    if (nblk > 0) {
        if ((e = check_hip(launch_quantize(L, c->P, k, v, src_tokens, src, nblk * (L.R / L.G), st.Lq, bh0, nbh, s),
                           "quantize")))
            return e;
        st.Lq += (int)(nblk * L.R);
        src += nblk * L.R;
        rem -= nblk * L.R;
    }
    // 4. the remainder starts a new residual
    if (rem > 0) {
        if ((e = check_hip(launch_copy_tokens(L, k, v, src_tokens, src, c->P.kres, c->P.vres, L.R, 0, rem,
                                              bh0, nbh, s),
                           "append")))
            return e;
        st.r = (int)rem;
    }
    return KVQ_OK;
}

int64_t max_len(const kvq_cache* c) { return *std::max_element(c->len.begin(), c->len.end()); }

// Paged records: gives every sequence the pages its key groups need once it holds
// new_len[b] tokens, from the pool's free pages, and writes the new table entries
// to the device (stream-ordered before the flushes that use them).  Fails, with
// nothing changed, when the pool has too few free pages.
kvq_status reserve_pages(kvq_cache* c, const std::vector<int64_t>& new_len, hipStream_t s) {
    const Layout& L = c->L;
    if (L.lp < 0) return KVQ_OK;
    std::vector<int> need((size_t)L.B);
    int64_t total = 0;
    for (int b = 0; b < L.B; ++b) {
        const int64_t groups = slice_state(new_len[b], L.S, L.R, L.Qf).Lq / L.G;
        need[b] = (int)((groups + (1 << L.lp) - 1) >> L.lp);
        total += std::max(0, need[b] - c->n_pages[b]);
    }
    if (total > (int64_t)c->free_pages.size())
        return fail(KVQ_ERR_CAPACITY, "the append needs %lld more pages, the pool has %zu free", (long long)total,
                    c->free_pages.size());
    std::vector<int> idx, val;
    for (int b = 0; b < L.B; ++b) {
        while (c->n_pages[b] < need[b]) {
            const int page = c->free_pages.back();
            c->free_pages.pop_back();
            const int i = (int)(b * L.max_pages + c->n_pages[b]);
            c->table[(size_t)i] = page;
            idx.push_back(i);
            val.push_back(page);
            c->n_pages[b] += 1;
        }
    }
    if (idx.empty()) return KVQ_OK;
    return check_hip(launch_set_entries(c->P.table, idx.data(), val.data(), (int)idx.size(), s), "append");
}

// After an append: back to the uniform state when every sequence has the same
// length; otherwise the state of the longest sequence, with the device lengths
// rewritten (write_lengths) or advanced by the caller.
kvq_status settle(kvq_cache* c, bool write_lengths, hipStream_t s) {
    const int64_t mx = max_len(c);
    const bool equal = *std::min_element(c->len.begin(), c->len.end()) == mx;
    const SliceState st = slice_state(mx, c->L.S, c->L.R, c->L.Qf);
    c->nS = st.nS, c->Lq = st.Lq, c->r = st.r;
    if (equal) {
        c->ragged = false;
        return KVQ_OK;
    }
    c->ragged = true;
    if (write_lengths) {
        kvq_status e = check_hip(launch_set_lengths(c->L, c->base_len, c->len.data(), s), "append");
        if (e != KVQ_OK) return e;
        c->len_delta = 0;
    }
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_append(kvq_cache* c, const void* k, const void* v, int64_t n_new, void* stream) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    if (n_new < 0) return fail(KVQ_ERR_INVALID_ARG, "n_new must be >= 0");
    if (n_new == 0) return ok();
    if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k or v is NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    const Layout& L = c->L;
    const int64_t total = max_len(c);
    if (n_new > L.max_tokens - total)
        return fail(KVQ_ERR_CAPACITY, "append of %lld tokens exceeds max_tokens %lld (holding %lld)",
                    (long long)n_new, (long long)L.max_tokens, (long long)total);
    hipStream_t s = (hipStream_t)stream;
    kvq_status st;
    {
        std::vector<int64_t> to(c->len);
        for (auto& n : to) n += n_new;
        if ((st = reserve_pages(c, to, s)) != KVQ_OK) return st;
    }
    if (!c->ragged) {
        SliceState ss{(int)c->nS, (int)c->Lq, (int)c->r};
        if ((st = append_slices(c, k, v, n_new, n_new, 0, L.BH, ss, s)) != KVQ_OK) return st;
        c->nS = ss.nS, c->Lq = ss.Lq, c->r = ss.r;
        for (auto& n : c->len) n += n_new;
        return ok();
    }
    if (n_new == 1) {
        // every sequence's token to its own sink slot or residual row, then the
        // flush of each sequence whose residual is now full
        if ((st = check_hip(launch_copy_one_ragged(L, c->P, k, v, Ragged{c->base_len, c->len_delta}, s),
                            "append")))
            return st;
        for (int b = 0; b < L.B; ++b) {
            const SliceState ss = slice_state(c->len[b], L.S, L.R, L.Qf);
            if (c->len[b] >= L.S && ss.r + 1 == L.R) {
                if ((st = check_hip(launch_flush(L, c->P, ss.Lq, (int64_t)b * L.Hkv, L.Hkv, s), "flush")))
                    return st;
            }
            c->len[b] += 1;
        }
        c->len_delta += 1;
        return (st = settle(c, false, s)) != KVQ_OK ? st : ok();
    }
    // several tokens: sequence by sequence
    for (int b = 0; b < L.B; ++b) {
        SliceState ss = slice_state(c->len[b], L.S, L.R, L.Qf);
        if ((st = append_slices(c, k, v, n_new, n_new, (int64_t)b * L.Hkv, L.Hkv, ss, s)) != KVQ_OK) return st;
        c->len[b] += n_new;
    }
    return (st = settle(c, true, s)) != KVQ_OK ? st : ok();
}

kvq_status kvq_append_ragged(kvq_cache* c, const void* k, const void* v, const int32_t* n_new, int64_t n_max,
                             void* stream) {
    if (!c || !n_new) return fail(KVQ_ERR_INVALID_ARG, "cache or n_new is NULL");
    if (n_max < 0) return fail(KVQ_ERR_INVALID_ARG, "n_max must be >= 0");
    const Layout& L = c->L;
    bool any = false;
    for (int b = 0; b < L.B; ++b) {
        if (n_new[b] < 0 || n_new[b] > n_max)
            return fail(KVQ_ERR_INVALID_ARG, "n_new[%d] = %d is outside [0, n_max = %lld]", b, n_new[b],
                        (long long)n_max);
        if (n_new[b] > L.max_tokens - c->len[b])
            return fail(KVQ_ERR_CAPACITY, "append of %d tokens to sequence %d exceeds max_tokens %lld (holding %lld)",
                        n_new[b], b, (long long)L.max_tokens, (long long)c->len[b]);
        any |= n_new[b] > 0;
    }
    if (!any) return ok();
    if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k or v is NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    kvq_status st;
    {
        std::vector<int64_t> to(c->len);
        for (int b = 0; b < L.B; ++b) to[(size_t)b] += n_new[b];
        if ((st = reserve_pages(c, to, s)) != KVQ_OK) return st;
    }
    for (int b = 0; b < L.B; ++b) {
        if (n_new[b] == 0) continue;
        SliceState ss = slice_state(c->len[b], L.S, L.R, L.Qf);
        if ((st = append_slices(c, k, v, n_new[b], n_max, (int64_t)b * L.Hkv, L.Hkv, ss, s)) != KVQ_OK) return st;
        c->len[b] += n_new[b];
    }
    return (st = settle(c, true, s)) != KVQ_OK ? st : ok();
}

kvq_status kvq_release_sequence(kvq_cache* c, int32_t b, void* stream) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    const Layout& L = c->L;
    if (b < 0 || b >= L.B) return fail(KVQ_ERR_INVALID_ARG, "sequence %d is outside [0, %d)", b, L.B);
    if (L.lp >= 0) {
        for (int i = c->n_pages[b] - 1; i >= 0; --i) {
            int& e = c->table[(size_t)(b * L.max_pages + i)];
            c->free_pages.push_back(e);
            e = -1;
        }
        c->n_pages[b] = 0;
    }
    c->len[b] = 0;
    kvq_status st = settle(c, true, (hipStream_t)stream);
    return st != KVQ_OK ? st : ok();
}

kvq_status kvq_pool_free_pages(const kvq_cache* c, int64_t* free_pages) {
    if (!c || !free_pages) return fail(KVQ_ERR_INVALID_ARG, "cache or free_pages is NULL");
    *free_pages = (int64_t)c->free_pages.size();
    return ok();
}

kvq_status kvq_seq_lengths(const kvq_cache* c, int64_t* lens) {
    if (!c || !lens) return fail(KVQ_ERR_INVALID_ARG, "cache or lens is NULL");
    for (int b = 0; b < c->L.B; ++b) lens[b] = c->len[b];
    return ok();
}

kvq_status kvq_decode_workspace_bytes(const kvq_cache* c, size_t* bytes) {
    if (!c || !bytes) return fail(KVQ_ERR_INVALID_ARG, "NULL argument");
    *bytes = decode_workspace_bytes(c->L, c->nsplit_cap);
    return ok();
}

}  // extern "C"

namespace {

// The checks of a decode call that do not involve the workspace.
kvq_status decode_checks(const kvq_cache* c, const void* q, const float* out, const float* lse) {
    if (!c || !q || !out) return fail(KVQ_ERR_INVALID_ARG, "cache, q or out is NULL");
    if (!aligned(q, 4) || !aligned(out, 4) || (lse && !aligned(lse, 4)))
        return fail(KVQ_ERR_INVALID_ARG, "misaligned q, out or lse");
    if (*std::min_element(c->len.begin(), c->len.end()) == 0)
        return fail(KVQ_ERR_INVALID_ARG, c->ragged ? "attention on an empty sequence" : "attention on an empty cache");
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(kvq_cache* c, const void* q, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
    kvq_status st = decode_checks(c, q, out, lse);
    if (st != KVQ_OK) return st;
    if (!ws) return fail(KVQ_ERR_INVALID_ARG, "ws is NULL");
    if (!aligned(ws, 256)) return fail(KVQ_ERR_INVALID_ARG, "misaligned ws");
    const size_t need = decode_workspace_bytes(c->L, c->nsplit_cap);
    if (ws_bytes < need)
        return fail(KVQ_ERR_BUFFER_TOO_SMALL, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
    DecodeRequest rq;
    if (c->ragged) rq.rg = Ragged{c->base_len, c->len_delta};
    rq.Lq = c->Lq;
    rq.nS = c->nS;
    rq.r = c->r;
    rq.split_tokens = c->split_tokens;
    rq.num_cu = c->num_cu;
    rq.nsplit_cap = c->nsplit_cap;
    rq.ev_start = c->ev_start;
    rq.ev_stop = c->ev_stop;
    st = check_hip(launch_decode(c->L, c->P, rq, q, out, lse, ws, c->sm_scale, (hipStream_t)stream), "decode");
    if (st != KVQ_OK) return st;
    return ok();
}

kvq_status kvq_decode_attention_static(kvq_cache* c, const void* q, float* out, float* lse, void* stream) {
    kvq_status st = decode_checks(c, q, out, lse);
    if (st != KVQ_OK) return st;
    const size_t need = decode_workspace_bytes(c->L, c->nsplit_cap);
    if (need > kStaticScratchBytes)
        return fail(KVQ_ERR_BUFFER_TOO_SMALL, "this cache's decode needs %zu bytes of scratch; the static "
                    "scratch holds %zu (use kvq_decode_attention with a workspace)", need, kStaticScratchBytes);
    void* ws = nullptr;
    if ((st = check_hip(static_scratch((hipStream_t)stream, &ws), "static scratch")) != KVQ_OK) return st;
    return kvq_decode_attention(c, q, out, lse, ws, need, stream);
}

kvq_status kvq_append_decode(kvq_cache* c, const void* k, const void* v, const void* q, float* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!c || !k || !v || !q || !out || !ws)
        return fail(KVQ_ERR_INVALID_ARG, "cache, k, v, q, out or ws is NULL");
    const Layout& L = c->L;
    // Everything either path checks is checked here, before anything is enqueued:
    // the two-call path below must not append the token and then fail its decode.
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    if (!aligned(q, 4) || !aligned(out, 4) || (lse && !aligned(lse, 4)) || !aligned(ws, 256))
        return fail(KVQ_ERR_INVALID_ARG, "misaligned q, out, lse or ws");
    if (1 > L.max_tokens - max_len(c))
        return fail(KVQ_ERR_CAPACITY, "append of 1 token exceeds max_tokens %lld", (long long)L.max_tokens);
    {
        const size_t need = decode_workspace_bytes(L, c->nsplit_cap);
        if (ws_bytes < need)
            return fail(KVQ_ERR_BUFFER_TOO_SMALL, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
    }
    // A token that lands in a sink slot or fills the residual (flush), in any
    // sequence, takes the two-call path; every other token is appended inside the
    // decode launch (for sequences of different lengths, each at its own row).
    bool fused = true;
    if (c->ragged) {
        for (int b = 0; b < L.B && fused; ++b) {
            const SliceState ss = slice_state(c->len[b], L.S, L.R, L.Qf);
            fused = c->len[b] >= L.S && ss.r + 1 < L.R;
        }
    } else {
        fused = c->nS >= L.S && c->r + 1 < L.R;
    }
    if (!fused) {
        // The decode needs every sequence non-empty after the append: it is (one more token each).
        kvq_status st = kvq_append(c, k, v, 1, stream);
        if (st != KVQ_OK) return st;
        return kvq_decode_attention(c, q, out, lse, ws, ws_bytes, stream);
    }
    DecodeRequest rq;
    rq.Lq = c->Lq;
    rq.nS = c->nS;
    rq.r = c->r + 1;  // the state after the append (no sequence flushes)
    if (c->ragged) rq.rg = Ragged{c->base_len, c->len_delta + 1};
    rq.split_tokens = c->split_tokens;
    rq.num_cu = c->num_cu;
    rq.nsplit_cap = c->nsplit_cap;
    rq.knew = k;
    rq.vnew = v;
    rq.ev_start = c->ev_start;
    rq.ev_stop = c->ev_stop;
    kvq_status st = check_hip(launch_decode(L, c->P, rq, q, out, lse, ws, c->sm_scale, (hipStream_t)stream),
                              "append_decode");
    if (st != KVQ_OK) return st;
    for (auto& n : c->len) n += 1;
    if (c->ragged) {
        c->len_delta += 1;
        return (st = settle(c, false, (hipStream_t)stream)) != KVQ_OK ? st : ok();
    }
    c->r += 1;
    return ok();
}

kvq_status kvq_dequantize(const kvq_cache* c, float* k_out, float* v_out, void* stream) {
    if (!c || !k_out || !v_out) return fail(KVQ_ERR_INVALID_ARG, "NULL argument");
    kvq_status st = check_hip(launch_dequantize(c->L, c->P, c->nS, c->Lq, c->r, k_out, v_out,
                                                c->ragged ? Ragged{c->base_len, c->len_delta} : Ragged{},
                                                (hipStream_t)stream),
                              "dequantize");
    if (st != KVQ_OK) return st;
    return ok();
}

kvq_status kvq_export(const kvq_cache* c, uint8_t* k_codes, float* k_scale, float* k_zero,
                      uint8_t* v_codes, float* v_scale, float* v_zero, void* stream) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    kvq_status st = check_hip(launch_export(c->L, c->P, c->Lq, k_codes, k_scale, k_zero, v_codes,
                                            v_scale, v_zero,
                                            c->ragged ? Ragged{c->base_len, c->len_delta} : Ragged{},
                                            (hipStream_t)stream),
                              "export");
    if (st != KVQ_OK) return st;
    return ok();
}

kvq_status kvq_export_outliers(const kvq_cache* c, uint8_t* k_idx, float* k_val, uint8_t* v_idx, float* v_val,
                               void* stream) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    if (!c->L.outliers) return fail(KVQ_ERR_INVALID_ARG, "the cache keeps no outliers");
    kvq_status st = check_hip(launch_export_outliers(c->L, c->P, c->Lq, k_idx, k_val, v_idx, v_val,
                                                     c->ragged ? Ragged{c->base_len, c->len_delta} : Ragged{},
                                                     (hipStream_t)stream),
                              "export_outliers");
    if (st != KVQ_OK) return st;
    return ok();
}

kvq_status kvq_cache_state(const kvq_cache* c, int64_t* n_tokens, int64_t* n_sink, int64_t* n_quant,
                           int64_t* n_resid) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    if (n_tokens) *n_tokens = c->nS + c->Lq + c->r;
    if (n_sink) *n_sink = c->nS;
    if (n_quant) *n_quant = c->Lq;
    if (n_resid) *n_resid = c->r;
    return ok();
}

kvq_status kvq_set_split_tokens(kvq_cache* c, int64_t tokens_per_split) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    if (tokens_per_split < 0) return fail(KVQ_ERR_INVALID_ARG, "tokens_per_split must be >= 0");
    c->split_tokens = tokens_per_split;
    return ok();
}

kvq_status kvq_set_timing_events(kvq_cache* c, void* start_event, void* stop_event) {
    if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(KVQ_ERR_INVALID_ARG, "start_event and stop_event must both be set or both be NULL");
    c->ev_start = static_cast<hipEvent_t>(start_event);
    c->ev_stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

kvq_status kvq_stream_read_probe(const void* buf, size_t bytes, int32_t blocks_per_cu, uint32_t* sink,
                                 void* stream) {
    if (!buf || !sink) return fail(KVQ_ERR_INVALID_ARG, "buf or sink is NULL");
    if (!aligned(buf, 16) || !aligned(sink, 4) || bytes % 16 != 0)
        return fail(KVQ_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a multiple of 16");
    if (blocks_per_cu < 1 || blocks_per_cu > 64) return fail(KVQ_ERR_INVALID_ARG, "blocks_per_cu must be in [1, 64]");
    if (bytes == 0) return ok();
    int dev = 0, ncu = 0;
    kvq_status st;
    if ((st = check_hip(hipGetDevice(&dev), "hipGetDevice")) != KVQ_OK) return st;
    if ((st = check_hip(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev),
                        "hipDeviceGetAttribute")) != KVQ_OK)
        return st;
    const int blocks = std::max(ncu, 1) * blocks_per_cu;
    st = check_hip(launch_stream_read(buf, (int64_t)(bytes / 16), blocks, sink, (hipStream_t)stream),
                   "stream_read_probe");
    if (st != KVQ_OK) return st;
    return ok();
}

const char* kvq_last_error(void) { return g_err; }

}  // extern "C"
