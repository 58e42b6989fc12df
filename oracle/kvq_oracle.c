/*
 * kvq_oracle.c -- plain, slow CPU oracle for low-bit KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library: no headers, no helpers, no tables.
 *
 * What it computes, and where the pages state it:
 *   - the asymmetric min-max group quantizer and its inverse
 *       scale = (max - min) / (2^n - 1), zero = round(-min / scale)
 *         ("KV Cache的Int4量化：如何解决Attention Sink导致的量化精度崩塌问题",
 *          section 2 "量化基础：线性量化", Min-Max bullet; and
 *          "Atom: Low-bit Quantization for Efficient and Accurate LLM Serving",
 *          section 三 "核心公式", asymmetric parameters with clip factor c = 1)
 *       code = clamp(round(x / scale) + zero, 0, 2^n - 1)
 *         (Atom review, section 三 "核心公式", quantized-tensor formula)
 *       x' = (code - zero) * scale
 *         (Int4 KV-cache post, section 2, dequantization formula)
 *   - code widths n = 2, 4 and 8 (8-bit codes: the per-layer INT8 / INT4 mixed
 *     precision of the Int4 KV-cache post, section 5.1)
 *   - the symmetric variant of the same quantizer (codec 1)
 *       scale = 2 max|x| / (2^n - 1), signed code clamp(round(x / scale),
 *       -2^(n-1), 2^(n-1) - 1)
 *         (Atom review, section 三 "核心公式", symmetric simplification, c = 1),
 *       stored as the unsigned code signed + 2^(n-1), i.e. zero = 2^(n-1), so
 *       the same dequantization applies
 *   - the KIVI cache layout: keys grouped per channel over G tokens, values
 *     per token, newest tokens in a full-precision residual that is quantized
 *     and appended once it holds R tokens, then emptied
 *       ("LLM系列：KVCache量化1 KIVI: A Tuning-Free Asymmetric 2bit Quantiz",
 *        section 1 "KIVI", key-cache split into grouped part and residual)
 *   - head-granular keys (key_axis 1): each token's key, the D channels of one
 *     attention head, is one asymmetric group, like a value group of G_V = D
 *       (Atom review, section 三, model-components table, KV-cache row: low-bit
 *        asymmetric quantization at attention-head granularity)
 *   - LogQuant's log-sparse retention (W > 0): the full-precision part holds
 *     at most 3W tokens; when full, its oldest 2W tokens are thinned to every
 *     other one, the thinned-out W are quantized, and the newest W stay
 *       ("Resumo Técnico: LogQuant", Metodologia item 2, window configuration,
 *        selection scheme, full-precision reserve and dynamic adjustment; item 4:
 *        quantized and full-precision tokens may be concatenated in any order)
 *   - KVQuant's per-vector dense-and-sparse quantization (outliers = 1): in every
 *     quantization vector the element of largest magnitude is an outlier, kept
 *     at full precision beside the codes; the vector's scale and zero point come
 *     from the other elements ("LLM系列：KVCache量化1 KIVI…" page, section 3
 *     "KVQuant", item (4): a small share of numeric outliers, e.g. 1%, stays
 *     unquantized in a separate sparse matrix)
 *   - attention softmax(q K^T / sqrt(d)) V over every cached token
 *       (Int4 KV-cache post, section 3, attention formula; KIVI notes, section 1,
 *        logits as the concatenation of the grouped and residual parts;
 *        "Resumo Técnico: LogQuant", Metodologia item 4: token order does not
 *        change the result).
 *
 * Precision.  The codec is an encoding, so it is followed step by step in
 * IEEE-754 binary32 with round-to-nearest-even per operation (build with
 * -ffp-contract=off, no fast-math, denormals kept): exactly one rounding per
 * written operation, in the written order.  Attention has a plain closed form
 * and is computed in binary64 from the exact fp32 dequantized values.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   round = round-half-to-even; codes unsigned in [0, 2^n - 1];
 *   code = clamp(rint(x/s) + z) in that order; clip factor c = 1;
 *   a group whose computed scale is 0 (max == min, or a range so small that
 *   range/(2^n-1) underflows) uses scale |min| (or 1 when min == 0);
 *   a zero point of -0 is stored as +0; zero points are integer-valued fp32
 *   and may fall outside [0, 2^n - 1];
 *   symmetric codec: max|x| from the group's min and max; a group whose scale
 *   computes to 0 uses max|x| (or 1 when the group is all zeros); the signed
 *   code range [-2^(n-1), 2^(n-1) - 1] is stored offset by 2^(n-1);
 *   the whole residual (R tokens, keys and values) is flushed when it reaches R;
 *   log-sparse retention: R = 3W; of each pair of the oldest 2W tokens the
 *   earlier one is quantized and the later one kept, so that the kept tokens
 *   thin out with their distance from the newest token; the W quantized tokens
 *   join the quantized part as W/G key groups in their order;
 *   the first S tokens of a sequence stay full precision for good (sinks);
 *   dense-and-sparse: one outlier per quantization vector (a key channel over G
 *   tokens, a token's G_V value channels), the element of largest |x|, the
 *   lowest index among equal magnitudes; it still receives a code, clamped like
 *   any other, but dequantizes to its exact value;
 *   query head h reads kv head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

/* ---------------------------------------------------------------------- */
/* group quantizer                                                         */
/* ---------------------------------------------------------------------- */

#define ORC_CODEC_ASYMMETRIC 0
#define ORC_CODEC_SYMMETRIC 1

/*
 * Quantize m values x[0], x[stride], ... to n-bit codes with the asymmetric
 * (codec 0) or symmetric (codec 1) quantizer, the scale and zero point taken
 * from every element but x[skip * stride] (skip = -1: from all; m >= 2 when
 * skipping).  Writes the group's scale and zero point and the codes q[0],
 * q[qstride], ... of all m elements.
 */
void orc_quant_group_skip(const float* x, int64_t m, int64_t stride, int bits, int codec, int64_t skip,
                          float* s_out, float* z_out, uint8_t* q, int64_t qstride)
{
    const int64_t first = skip == 0 ? 1 : 0;
    float mn = x[first * stride], mx = x[first * stride];
    for (int64_t i = first + 1; i < m; ++i) {
        if (i == skip) continue;
        float v = x[i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    const float qmax = (float)((1 << bits) - 1);  /* 2^n - 1, exact */
    if (codec == ORC_CODEC_SYMMETRIC) {
        const float amax = fabsf(mn) > fabsf(mx) ? fabsf(mn) : fabsf(mx);
        const float twice = 2.0f * amax;        /* exact */
        float ss = twice / qmax;
        if (ss == 0.0f) ss = (amax != 0.0f) ? amax : 1.0f;
        const float zz = (float)(1 << (bits - 1));  /* 2^(n-1): signed code + zz */
        for (int64_t i = 0; i < m; ++i) {
            float r = rintf(x[i * stride] / ss);
            if (r < -zz) r = -zz;
            if (r > zz - 1.0f) r = zz - 1.0f;
            q[i * qstride] = (uint8_t)(r + zz);
        }
        *s_out = ss;
        *z_out = zz;
        return;
    }
    float range = mx - mn;
    float s = range / qmax;
    if (mx == mn || s == 0.0f) {
        /* degenerate group: keep the closed forms with a nonzero scale */
        s = (mn != 0.0f) ? fabsf(mn) : 1.0f;
    }
    float negmn = -mn;
    float z = rintf(negmn / s);
    if (z == 0.0f) z = 0.0f; /* canonical +0 */
    for (int64_t i = 0; i < m; ++i) {
        float xi = x[i * stride];
        float r = rintf(xi / s);
        float t = r + z;
        if (t < 0.0f) t = 0.0f;
        if (t > qmax) t = qmax;
        q[i * qstride] = (uint8_t)t;
    }
    *s_out = s;
    *z_out = z;
}

void orc_quant_group(const float* x, int64_t m, int64_t stride, int bits, int codec,
                     float* s_out, float* z_out, uint8_t* q, int64_t qstride)
{
    orc_quant_group_skip(x, m, stride, bits, codec, -1, s_out, z_out, q, qstride);
}

/* The index of the element of largest magnitude (the lowest among equal ones). */
int64_t orc_outlier_index(const float* x, int64_t m, int64_t stride)
{
    int64_t best = 0;
    for (int64_t i = 1; i < m; ++i)
        if (fabsf(x[i * stride]) > fabsf(x[best * stride])) best = i;
    return best;
}

/* x' = (code - zero) * scale */
float orc_dequant(uint8_t q, float s, float z)
{
    float d = (float)q - z;
    return d * s;
}

/* ---------------------------------------------------------------------- */
/* cache state of one (sequence, kv-head) slice                            */
/* ---------------------------------------------------------------------- */

#define ORC_KEY_PER_CHANNEL 0
#define ORC_KEY_PER_TOKEN 1

typedef struct {
    int D, bits, codec, G, GV, R, S;
    int key_axis;                               /* ORC_KEY_PER_CHANNEL or ORC_KEY_PER_TOKEN */
    int W;                                      /* log window; 0: whole-residual flush */
    /* buffers owned by the caller */
    float* sink_k; float* sink_v;               /* [S, D]            */
    uint8_t* k_codes; float* k_scale; float* k_zero;   /* [Lq,D] [Lq/G,D], per token [Lq] */
    uint8_t* v_codes; float* v_scale; float* v_zero;   /* [Lq,D] [Lq,D/GV] */
    float* res_k; float* res_v;                 /* [R, D]            */
    int outliers;                               /* one per vector, or none */
    int32_t* ko_idx; float* ko_val;             /* [Lq/G, D]: token in group, value */
    int32_t* vo_idx; float* vo_val;             /* [Lq, D/GV]: channel in group, value */
    int64_t nS, Lq, r, flushes;
} orc_slice;

/*
 * Quantize m tokens (bk, bv: [m, D], m a multiple of G) and append them to the
 * quantized part.
 */
static void quantize_block(orc_slice* c, const float* bk, const float* bv, int m)
{
    const int D = c->D, G = c->G, GV = c->GV;
    const int nvg = D / GV;
    /* head-granular keys: one group per token over its D channels */
    if (c->key_axis == ORC_KEY_PER_TOKEN) {
        for (int t = 0; t < m; ++t) {
            const int64_t tok = c->Lq + t;
            orc_quant_group(bk + (int64_t)t * D, D, 1, c->bits, c->codec,
                            &c->k_scale[tok], &c->k_zero[tok], c->k_codes + tok * D, 1);
        }
    }
    /* keys: one group per channel over each run of G tokens */
    for (int j = 0; c->key_axis == ORC_KEY_PER_CHANNEL && j < m / G; ++j) {
        int64_t grp = c->Lq / G + j;
        for (int ch = 0; ch < D; ++ch) {
            const float* col = bk + (int64_t)j * G * D + ch;
            const int64_t o = c->outliers ? orc_outlier_index(col, G, D) : -1;
            orc_quant_group_skip(col, G, D, c->bits, c->codec, o,
                                 &c->k_scale[grp * D + ch], &c->k_zero[grp * D + ch],
                                 c->k_codes + (c->Lq + (int64_t)j * G) * D + ch, D);
            if (c->outliers) {
                c->ko_idx[grp * D + ch] = (int32_t)o;
                c->ko_val[grp * D + ch] = col[o * D];
            }
        }
    }
    /* values: one group per run of GV channels of each token */
    for (int t = 0; t < m; ++t) {
        int64_t tok = c->Lq + t;
        for (int h = 0; h < nvg; ++h) {
            const float* vec = bv + (int64_t)t * D + (int64_t)h * GV;
            const int64_t o = c->outliers ? orc_outlier_index(vec, GV, 1) : -1;
            orc_quant_group_skip(vec, GV, 1, c->bits, c->codec, o,
                                 &c->v_scale[tok * nvg + h], &c->v_zero[tok * nvg + h],
                                 c->v_codes + tok * D + (int64_t)h * GV, 1);
            if (c->outliers) {
                c->vo_idx[tok * nvg + h] = (int32_t)o;
                c->vo_val[tok * nvg + h] = vec[o];
            }
        }
    }
    c->Lq += m;
}

/* Quantize the full residual (R tokens) and append it to the quantized part. */
static void flush_residual(orc_slice* c)
{
    quantize_block(c, c->res_k, c->res_v, c->R);
    c->r = 0;
    c->flushes += 1;
}

/*
 * Log-sparse retention, the full-precision part holding 3W tokens: of the
 * oldest 2W (slots 0 .. 2W-1) the earlier token of each pair (slots 0, 2, ...)
 * is quantized and the later one (slots 1, 3, ...) kept; the kept W and then
 * the newest W (slots 2W .. 3W-1) form the new full-precision part.
 */
static void flush_log(orc_slice* c)
{
    const int D = c->D, W = c->W;
    float* bk = (float*)malloc(sizeof(float) * (size_t)W * D);
    float* bv = (float*)malloc(sizeof(float) * (size_t)W * D);
    float* keep_k = (float*)malloc(sizeof(float) * (size_t)2 * W * D);
    float* keep_v = (float*)malloc(sizeof(float) * (size_t)2 * W * D);
    for (int i = 0; i < W; ++i) {
        memcpy(bk + (size_t)i * D, c->res_k + (size_t)(2 * i) * D, sizeof(float) * D);
        memcpy(bv + (size_t)i * D, c->res_v + (size_t)(2 * i) * D, sizeof(float) * D);
        memcpy(keep_k + (size_t)i * D, c->res_k + (size_t)(2 * i + 1) * D, sizeof(float) * D);
        memcpy(keep_v + (size_t)i * D, c->res_v + (size_t)(2 * i + 1) * D, sizeof(float) * D);
    }
    memcpy(keep_k + (size_t)W * D, c->res_k + (size_t)2 * W * D, sizeof(float) * (size_t)W * D);
    memcpy(keep_v + (size_t)W * D, c->res_v + (size_t)2 * W * D, sizeof(float) * (size_t)W * D);
    quantize_block(c, bk, bv, W);
    memcpy(c->res_k, keep_k, sizeof(float) * (size_t)2 * W * D);
    memcpy(c->res_v, keep_v, sizeof(float) * (size_t)2 * W * D);
    c->r = 2 * W;
    c->flushes += 1;
    free(bk); free(bv); free(keep_k); free(keep_v);
}

/* Append one token: sink slot while sinks remain, else residual; flush at R. */
static void append_token(orc_slice* c, const float* k, const float* v)
{
    const int D = c->D;
    if (c->nS < c->S) {
        memcpy(c->sink_k + c->nS * D, k, sizeof(float) * D);
        memcpy(c->sink_v + c->nS * D, v, sizeof(float) * D);
        c->nS += 1;
        return;
    }
    memcpy(c->res_k + c->r * D, k, sizeof(float) * D);
    memcpy(c->res_v + c->r * D, v, sizeof(float) * D);
    c->r += 1;
    if (c->r == c->R) {
        if (c->W > 0) flush_log(c);
        else flush_residual(c);
    }
}

/*
 * Build the cache of one slice by appending n tokens (fp32 [n, D] each) one
 * at a time.  W = 0 flushes the whole residual at R tokens; W > 0 selects the
 * log-sparse retention, with R = 3W and W a multiple of G.  counts[0..3]
 * receive nS, Lq, r and the number of flushes.  Output buffers must hold the
 * sizes given above for the final Lq: with m = n - S tokens past the sinks,
 * R*floor(m/R), or with W > 0, 0 for m < R and W*(floor((m-R)/W) + 1) after.
 * outliers = 1 keeps one outlier per quantization vector: ko_idx, ko_val
 * [Lq/G, D] (token within the group, exact value), vo_idx, vo_val [Lq, D/GV]
 * (channel within the group, exact value); with outliers = 0 they are unused.
 * key_axis = ORC_KEY_PER_TOKEN quantizes each token's key as one group (k_scale,
 * k_zero [Lq]) instead of each channel over G tokens; it takes no outliers.
 * Returns 0, or -1 on an invalid configuration.
 */
int orc_build_slice(int D, int bits, int codec, int G, int GV, int R, int S, int W, int outliers,
                    int key_axis, const float* k_tok, const float* v_tok, int64_t n,
                    float* sink_k, float* sink_v,
                    uint8_t* k_codes, float* k_scale, float* k_zero,
                    uint8_t* v_codes, float* v_scale, float* v_zero,
                    float* res_k, float* res_v,
                    int32_t* ko_idx, float* ko_val, int32_t* vo_idx, float* vo_val, int64_t* counts)
{
    if (D <= 0 || G <= 0 || GV <= 0 || R <= 0 || S < 0 || n < 0) return -1;
    if (bits != 2 && bits != 4 && bits != 8) return -1;
    if (codec != ORC_CODEC_ASYMMETRIC && codec != ORC_CODEC_SYMMETRIC) return -1;
    if (R % G != 0 || D % GV != 0) return -1;
    if (W < 0 || (W > 0 && (R != 3 * W || W % G != 0))) return -1;
    if (outliers != 0 && (outliers != 1 || G < 2 || GV < 2)) return -1;
    if (key_axis != ORC_KEY_PER_CHANNEL && key_axis != ORC_KEY_PER_TOKEN) return -1;
    if (key_axis == ORC_KEY_PER_TOKEN && outliers) return -1;
    orc_slice c = {D, bits, codec, G, GV, R, S, key_axis, W, sink_k, sink_v, k_codes, k_scale, k_zero,
                   v_codes, v_scale, v_zero, res_k, res_v, outliers, ko_idx, ko_val, vo_idx, vo_val,
                   0, 0, 0, 0};
    for (int64_t t = 0; t < n; ++t)
        append_token(&c, k_tok + t * D, v_tok + t * D);
    counts[0] = c.nS; counts[1] = c.Lq; counts[2] = c.r; counts[3] = c.flushes;
    return 0;
}

/*
 * Dequantize one slice in storage order: sinks, then the quantized tokens in
 * the order they were quantized, then the full-precision part (chronological
 * order when whole residuals are flushed).  k_out, v_out: fp32 [nS+Lq+r, D].
 * key_axis selects the key scale / zero layout ([Lq/G, D], or [Lq] per token).
 */
void orc_dequant_slice(int D, int G, int GV, int key_axis, int64_t nS, int64_t Lq, int64_t r,
                       const float* sink_k, const float* sink_v,
                       const uint8_t* k_codes, const float* k_scale, const float* k_zero,
                       const uint8_t* v_codes, const float* v_scale, const float* v_zero,
                       const float* res_k, const float* res_v,
                       int outliers, const int32_t* ko_idx, const float* ko_val,
                       const int32_t* vo_idx, const float* vo_val,
                       float* k_out, float* v_out)
{
    const int nvg = D / GV;
    memcpy(k_out, sink_k, sizeof(float) * nS * D);
    memcpy(v_out, sink_v, sizeof(float) * nS * D);
    for (int64_t t = 0; t < Lq; ++t) {
        int64_t grp = t / G;
        for (int ch = 0; ch < D; ++ch) {
            const int64_t km = key_axis == ORC_KEY_PER_TOKEN ? t : grp * D + ch;
            k_out[(nS + t) * D + ch] = orc_dequant(k_codes[t * D + ch], k_scale[km], k_zero[km]);
            int h = ch / GV;
            v_out[(nS + t) * D + ch] = orc_dequant(v_codes[t * D + ch],
                                                   v_scale[t * nvg + h], v_zero[t * nvg + h]);
            /* outliers: their exact values */
            if (outliers && ko_idx[grp * D + ch] == t % G) k_out[(nS + t) * D + ch] = ko_val[grp * D + ch];
            if (outliers && vo_idx[t * nvg + h] == ch - h * GV) v_out[(nS + t) * D + ch] = vo_val[t * nvg + h];
        }
    }
    memcpy(k_out + (nS + Lq) * D, res_k, sizeof(float) * r * D);
    memcpy(v_out + (nS + Lq) * D, res_v, sizeof(float) * r * D);
}

/* ---------------------------------------------------------------------- */
/* attention                                                               */
/* ---------------------------------------------------------------------- */

/*
 * out = softmax(scale * q K^T) V and lse = log(sum(exp(scale * q K^T))) for one
 * query row over T tokens, in binary64.  The order of the tokens is immaterial.
 */
void orc_attention(const float* q, const float* K, const float* V, int64_t T, int D,
                   double scale, double* out, double* lse)
{
    double* sc = (double*)malloc(sizeof(double) * (T > 0 ? T : 1));
    double M = -INFINITY;
    for (int64_t j = 0; j < T; ++j) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += (double)q[c] * (double)K[j * D + c];
        sc[j] = dot * scale;
        if (sc[j] > M) M = sc[j];
    }
    double den = 0.0;
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    for (int64_t j = 0; j < T; ++j) {
        double w = exp(sc[j] - M);
        den += w;
        for (int c = 0; c < D; ++c) out[c] += w * (double)V[j * D + c];
    }
    for (int c = 0; c < D; ++c) out[c] /= den;
    *lse = M + log(den);
    free(sc);
}

/*
 * One decode step over n independent slices that share a cache state
 * (nS, Lq, r): dequantize each slice, then attend each of its g query heads.
 * Arrays are the per-slice arrays above stacked along a leading slice axis;
 * q is fp32 [n, g, D]; out [n, g, D] and lse [n, g] are binary64.
 * Slices are independent, so they are spread over OpenMP threads.
 */
void orc_decode_slices(int64_t n, int g, int D, int G, int GV, int key_axis,
                       int64_t nS, int64_t Lq, int64_t r, double scale,
                       const float* sink_k, const float* sink_v,
                       const uint8_t* k_codes, const float* k_scale, const float* k_zero,
                       const uint8_t* v_codes, const float* v_scale, const float* v_zero,
                       const float* res_k, const float* res_v,
                       int outliers, const int32_t* ko_idx, const float* ko_val,
                       const int32_t* vo_idx, const float* vo_val,
                       const float* q, double* out, double* lse)
{
    const int64_t T = nS + Lq + r;
    const int64_t nvg = D / GV;
    const int64_t nkm = key_axis == ORC_KEY_PER_TOKEN ? Lq : (Lq / G) * D;  /* key scales per slice */
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        float* kf = (float*)malloc(sizeof(float) * (T > 0 ? T : 1) * D);
        float* vf = (float*)malloc(sizeof(float) * (T > 0 ? T : 1) * D);
        orc_dequant_slice(D, G, GV, key_axis, nS, Lq, r,
                          sink_k + i * nS * D, sink_v + i * nS * D,
                          k_codes + i * Lq * D, k_scale + i * nkm, k_zero + i * nkm,
                          v_codes + i * Lq * D, v_scale + i * Lq * nvg, v_zero + i * Lq * nvg,
                          res_k + i * r * D, res_v + i * r * D, outliers,
                          ko_idx + (outliers ? i * (Lq / G) * D : 0), ko_val + (outliers ? i * (Lq / G) * D : 0),
                          vo_idx + (outliers ? i * Lq * nvg : 0), vo_val + (outliers ? i * Lq * nvg : 0), kf, vf);
        for (int h = 0; h < g; ++h)
            orc_attention(q + (i * g + h) * D, kf, vf, T, D, scale,
                          out + (i * g + h) * D, lse + i * g + h);
        free(kf);
        free(vf);
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel regions above (timing of the oracle only; n >= 1). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
