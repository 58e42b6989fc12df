"""Second, independent formulation of the oracle for tiny inputs (test infrastructure).

Pure Python over numpy scalars: binary32 scalar arithmetic for the codec
(numpy's float32 scalar operations round once per operation, to nearest even)
and math.fsum-free explicit float64 loops for attention.  It exists to
cross-check ``kvq_oracle.c`` on inputs small enough for Python loops; it does
not import that library.

Sources: asymmetric min-max parameters and the clamp-round code
("Atom: Low-bit Quantization for Efficient and Accurate LLM Serving",
section 三 "核心公式"); dequantization (q - zero) * scale
("KV Cache的Int4量化：如何解决Attention Sink导致的量化精度崩塌问题", section 2);
attention softmax(q K^T / sqrt(d)) V (same post, section 3).
"""
from __future__ import annotations

import math

import numpy as np

f32 = np.float32


def quant_group(values, bits: int, codec: int = 0, range_of=None):
    """Returns (scale, zero, codes) with one binary32 rounding per operation.

    codec 0: asymmetric min-max; codec 1: symmetric, scale 2 max|x| / (2^n - 1),
    signed code clamp(rint(x / scale), -2^(n-1), 2^(n-1) - 1) stored plus 2^(n-1)
    (Atom review, section 三 "核心公式", symmetric simplification, c = 1).
    range_of: the values whose min and max set the scale (default: values).
    """
    xs = [f32(v) for v in values]
    rs = xs if range_of is None else [f32(v) for v in range_of]
    mn = min(rs)
    mx = max(rs)
    qmax = f32((1 << bits) - 1)
    if codec == 1:
        amax = max(abs(mn), abs(mx))
        s = f32(f32(f32(2) * amax) / qmax)
        if s == f32(0):
            s = amax if amax != f32(0) else f32(1)
        half = 1 << (bits - 1)
        codes = []
        for x in xs:
            r = int(np.rint(f32(x / s)))
            codes.append(min(max(r, -half), half - 1) + half)
        return s, f32(half), codes
    s = f32(f32(mx - mn) / qmax)
    if mx == mn or s == f32(0):
        s = f32(abs(mn)) if mn != f32(0) else f32(1)
    z = f32(np.rint(f32(f32(-mn) / s)))
    if z == f32(0):
        z = f32(0.0)
    codes = []
    for x in xs:
        t = f32(f32(np.rint(f32(x / s))) + z)
        t = min(max(t, f32(0)), qmax)
        codes.append(int(t))
    return s, z, codes


def quant_group_sparse(values, bits: int, codec: int = 0):
    """KVQuant's per-vector dense-and-sparse split ("LLM系列：KVCache量化1 KIVI…"
    page, section 3, item (4)): the element of largest magnitude (first among
    equals) is the outlier; the others set the scale; every element gets a code.
    Returns (scale, zero, codes, outlier index)."""
    mags = [abs(float(v)) for v in values]
    o = mags.index(max(mags))
    s, z, codes = quant_group(values, bits, codec, range_of=[v for i, v in enumerate(values) if i != o])
    return s, z, codes, o


def dequant(code: int, s, z):
    return f32(f32(f32(code) - f32(z)) * f32(s))


def attention(q, K, V, scale: float):
    """Explicit-loop binary64 attention of one query row over the rows of K, V."""
    T = len(K)
    D = len(q)
    scores = []
    for j in range(T):
        acc = 0.0
        for c in range(D):
            acc += float(q[c]) * float(K[j][c])
        scores.append(acc * scale)
    m = max(scores)
    ws = [math.exp(s - m) for s in scores]
    den = sum(ws)
    out = [sum(ws[j] * float(V[j][c]) for j in range(T)) / den for c in range(D)]
    return np.array(out), m + math.log(den)


def build_slice(k_tok, v_tok, *, bits, k_group, v_group, residual, n_sink, codec=0, log_window=0,
                outliers=0, key_axis=0):
    """Token-by-token cache construction, written independently of the C oracle.

    log_window W > 0: LogQuant's log-sparse retention ("Resumo Técnico: LogQuant",
    Metodologia item 2).  The full-precision list holds up to residual = 3W
    tokens; when full, its first 2W entries are split into pairs, the first of
    each pair is quantized and the second kept, and the last W entries follow.

    outliers = 1: dense-and-sparse groups (quant_group_sparse); an outlier
    dequantizes to its own value.

    key_axis = 1: head-granular keys ("Atom…" review, section 三, model-components
    table, KV-cache row): every token's key row is one group, as a value row is
    with v_group equal to the row length; k_meta then holds one [(s, z)] per token.

    Returns dict with lists: sinks, quantized (dequantized K', V' rows in the
    order they were quantized), residual rows, codes and metadata, outliers
    (k_out per key block: [(token, value)] per channel; v_out per token:
    [(channel, value)] per value group), and the flush count.
    """
    D = len(k_tok[0])
    sinks_k, sinks_v, res_k, res_v = [], [], [], []
    qk_rows, qv_rows = [], []
    k_codes, v_codes, k_meta, v_meta = [], [], [], []
    k_out, v_out = [], []
    flushes = 0
    for kt, vt in zip(k_tok, v_tok):
        if len(sinks_k) < n_sink:
            sinks_k.append(list(kt))
            sinks_v.append(list(vt))
            continue
        res_k.append(list(kt))
        res_v.append(list(vt))
        if len(res_k) < residual:
            continue
        flushes += 1
        if log_window:
            W = log_window
            out_k, out_v = res_k[0:2 * W:2], res_v[0:2 * W:2]
            res_k = res_k[1:2 * W:2] + res_k[2 * W:]
            res_v = res_v[1:2 * W:2] + res_v[2 * W:]
        else:
            out_k, out_v = res_k, res_v
            res_k, res_v = [], []
        # head-granular keys: each quantized token's key row is one group
        if key_axis:
            for row in out_k:
                s, z, q = quant_group(row, bits, codec)
                qk_rows.append([dequant(code, s, z) for code in q])
                k_codes.append(list(q))
                k_meta.append([(s, z)])
        # keys: per channel over each run of k_group tokens
        for j0 in range(0, len(out_k) if not key_axis else 0, k_group):
            block = out_k[j0:j0 + k_group]
            rows = [[None] * D for _ in block]
            crow = [[0] * D for _ in block]
            meta, outs = [], []
            for c in range(D):
                col = [row[c] for row in block]
                if outliers:
                    s, z, q, o = quant_group_sparse(col, bits, codec)
                    outs.append((o, f32(col[o])))
                else:
                    (s, z, q), o = quant_group(col, bits, codec), None
                meta.append((s, z))
                for i, code in enumerate(q):
                    rows[i][c] = f32(col[i]) if i == o else dequant(code, s, z)
                    crow[i][c] = code
            qk_rows.extend(rows)
            k_codes.extend(crow)
            k_meta.append(meta)
            k_out.append(outs)
        # values: per token, per run of v_group channels
        for row in out_v:
            out, crow, meta, outs = [], [], [], []
            for h in range(0, D, v_group):
                vec = row[h:h + v_group]
                if outliers:
                    s, z, q, o = quant_group_sparse(vec, bits, codec)
                    outs.append((o, f32(vec[o])))
                else:
                    (s, z, q), o = quant_group(vec, bits, codec), None
                meta.append((s, z))
                out.extend(f32(vec[i]) if i == o else dequant(code, s, z) for i, code in enumerate(q))
                crow.extend(q)
            qv_rows.append(out)
            v_codes.append(crow)
            v_meta.append(meta)
            v_out.append(outs)
    return dict(sinks_k=sinks_k, sinks_v=sinks_v, qk=qk_rows, qv=qv_rows,
                res_k=res_k, res_v=res_v, k_codes=k_codes, v_codes=v_codes,
                k_meta=k_meta, v_meta=v_meta, k_out=k_out, v_out=v_out, flushes=flushes)
