"""Oracle: softmax attention in binary64 over dequantised pages, for decode,
verify and chunked prefill, plus the log-sum-exp merge of partial results.
Test infrastructure only (see the package docstring).

[RDNA4] "Stream-optimized speculative decoding": paged decode attention is
extended to verify batches (1 + n draft tokens, causally ordered among
themselves); "Online Log-Sum-Exp prefill & pipelined prefetch": chunked
prefill over pages with partial results accumulated by online LSE.
[STREAM] step ④: the streaming path runs flash attention over Q8_0 K / Q4_0 V.
The plain definition is written out (no tiling, no online rescaling): scores
s_j = scale * q . Khat_j over the visible keys, o = sum softmax(s)_j Vhat_j,
lse = max s + ln sum exp(s - max s), with an empty key set giving o = 0 and
lse = -inf.
"""
import numpy as np

from .quant import (HEAD_DIM, PAGE_TOKENS, BLOCK, N_BLOCKS, unpack_k_record,
                    unpack_v_record, unpack_v8_record, values_are_q8, dequantize_keys,
                    q8_0_dequantize,
                    q4_0_dequantize)


def dequant_page(k_records, v_records):
    """Dequantised keys and values (binary64, exact) of page records.
    k_records uint8 [..., 34816] (Q8_0 keys), [..., 18432] (Q4_0 keys) or
    [..., 24576] (Q5_1 keys),
    v_records uint8 [..., 18432] (Q4_0) or
    [..., 34816] (Q8_0) -> (Khat [..., 128, 256], Vhat [..., 128, 256])."""
    v8 = values_are_q8(v_records)
    vc, vb = (unpack_v8_record if v8 else unpack_v_record)(v_records)
    lead = vc.shape[:-2]
    shp = lead + (PAGE_TOKENS, N_BLOCKS, BLOCK)
    # unwritten slots may hold any bytes (inf/nan scales); callers drop them
    with np.errstate(invalid="ignore", over="ignore"):
        khat = dequantize_keys(k_records)
        vdq = q8_0_dequantize if v8 else q4_0_dequantize
        vhat = vdq(vc.reshape(shp), vb).reshape(lead + (PAGE_TOKENS, HEAD_DIM))
    return khat, vhat


def gather_keys(k_pool, v_pool, page_table, n_logical_pages, head, pages, kv_len):
    """Dequantised keys/values and positions of the tokens (< kv_len) on the
    listed logical pages of one KV head, in list order. A listed page outside
    [0, n_logical_pages), or whose physical page is outside the pool, is
    skipped. Returns (Khat [n, 256], Vhat [n, 256], pos int64 [n])."""
    n_phys = k_pool.shape[0]
    pages = np.asarray(pages, np.int64)
    ok = (pages >= 0) & (pages < n_logical_pages)
    pages = pages[ok]
    phys = np.asarray(page_table, np.int64)[pages]
    ok = (phys >= 0) & (phys < n_phys)
    pages, phys = pages[ok], phys[ok]
    if pages.size == 0:
        z = np.zeros((0, HEAD_DIM))
        return z, z, np.zeros(0, np.int64)
    khat, vhat = dequant_page(k_pool[phys, head], v_pool[phys, head])
    pos = (pages[:, None] * PAGE_TOKENS + np.arange(PAGE_TOKENS)[None, :]).reshape(-1)
    khat = khat.reshape(-1, HEAD_DIM)
    vhat = vhat.reshape(-1, HEAD_DIM)
    keep = pos < kv_len
    return khat[keep], vhat[keep], pos[keep]


def attend_rows(q_rows, khat, vhat, pos, limits, scale):
    """Softmax attention of query rows over a key set, in binary64.
    q_rows [R, 256]; key j is visible to row r iff pos[j] <= limits[r].
    Returns (o [R, 256], lse [R]) with natural-log lse."""
    q = np.asarray(q_rows, np.float64)
    R = q.shape[0]
    o = np.zeros((R, HEAD_DIM), np.float64)
    lse = np.full(R, -np.inf, np.float64)
    if khat.shape[0] == 0:
        return o, lse
    s = float(scale) * (q @ khat.T)                              # [R, n]
    visible = pos[None, :] <= np.asarray(limits, np.int64)[:, None]
    for r in range(R):
        sr = s[r][visible[r]]
        if sr.size == 0:
            continue
        m = sr.max()
        w = np.exp(sr - m)
        l_ = w.sum()
        o[r] = (w @ vhat[visible[r]]) / l_
        lse[r] = m + np.log(l_)
    return o, lse


def decode(q, gqa, k_pool, v_pool, page_table, n_logical_pages, kv_len, scale,
           blocks=None, kv_heads=None):
    """kvattn_decode semantics. q float32 [n_q_tok, n_kv*gqa, 256]; query token t
    sits at kv_len - n_q_tok + t and sees keys at positions <= that.
    blocks None (dense: every page up to kv_len) or int [n_kv, n_blk] logical
    pages per KV head. kv_heads: subset of KV heads to compute (others NaN).
    Returns (out float64 [n_q_tok, n_heads, 256], lse float64 [n_q_tok, n_heads])."""
    q = np.asarray(q, np.float32)
    n_q_tok, n_heads, _ = q.shape
    n_kv = n_heads // gqa
    out = np.full((n_q_tok, n_heads, HEAD_DIM), np.nan)
    lse = np.full((n_q_tok, n_heads), np.nan)
    n_pages = (kv_len + PAGE_TOKENS - 1) // PAGE_TOKENS
    for h in (range(n_kv) if kv_heads is None else kv_heads):
        pages = np.arange(n_pages) if blocks is None else np.asarray(blocks)[h]
        khat, vhat, pos = gather_keys(k_pool, v_pool, page_table, n_logical_pages,
                                      h, pages, kv_len)
        rows = q[:, h * gqa:(h + 1) * gqa].reshape(n_q_tok * gqa, HEAD_DIM)
        limits = np.repeat(kv_len - n_q_tok + np.arange(n_q_tok), gqa)
        o, l_ = attend_rows(rows, khat, vhat, pos, limits, scale)
        out[:, h * gqa:(h + 1) * gqa] = o.reshape(n_q_tok, gqa, HEAD_DIM)
        lse[:, h * gqa:(h + 1) * gqa] = l_.reshape(n_q_tok, gqa)
    return out, lse


def prefill_chunk(q, gqa, k_pool, v_pool, page_table, n_logical_pages, pos0, scale,
                  tokens=None, kv_heads=None):
    """kvattn_prefill_chunk semantics. q float32 [chunk, n_kv*gqa, 256]; query
    token t sits at pos0 + t and sees keys at positions <= pos0 + t.
    tokens / kv_heads: subsets to compute (others NaN), for sampled checks.
    Returns (out float64 [chunk, n_heads, 256], lse float64 [chunk, n_heads])."""
    q = np.asarray(q, np.float32)
    chunk, n_heads, _ = q.shape
    n_kv = n_heads // gqa
    kv_len = pos0 + chunk
    toks = np.arange(chunk) if tokens is None else np.asarray(tokens, np.int64)
    out = np.full((chunk, n_heads, HEAD_DIM), np.nan)
    lse = np.full((chunk, n_heads), np.nan)
    n_pages = (kv_len + PAGE_TOKENS - 1) // PAGE_TOKENS
    for h in (range(n_kv) if kv_heads is None else kv_heads):
        khat, vhat, pos = gather_keys(k_pool, v_pool, page_table, n_logical_pages,
                                      h, np.arange(n_pages), kv_len)
        rows = q[toks][:, h * gqa:(h + 1) * gqa].reshape(-1, HEAD_DIM)
        limits = np.repeat(pos0 + toks, gqa)
        o, l_ = attend_rows(rows, khat, vhat, pos, limits, scale)
        out[toks, h * gqa:(h + 1) * gqa] = o.reshape(len(toks), gqa, HEAD_DIM)
        lse[toks, h * gqa:(h + 1) * gqa] = l_.reshape(len(toks), gqa)
    return out, lse


def merge_lse(o_parts, lse_parts):
    """Merge partial results by log-sum-exp, in binary64 ([RDNA4] online LSE).
    o_parts [S, rows, D], lse_parts [S, rows] -> (out [rows, D], lse [rows]).
    M = max_s lse_s; L = M + ln sum_s exp(lse_s - M); out = sum_s exp(lse_s - L) o_s.
    A part with lse = -inf contributes nothing; all -inf gives out 0, lse -inf."""
    o = np.asarray(o_parts, np.float64)
    ls = np.asarray(lse_parts, np.float64)
    S, rows = ls.shape
    out = np.zeros(o.shape[1:], np.float64)
    lse = np.full(rows, -np.inf)
    for r in range(rows):
        M = ls[:, r].max()
        if M == -np.inf:
            continue
        L = M + np.log(np.sum(np.exp(ls[:, r] - M)))
        w = np.exp(ls[:, r] - L)
        out[r] = w @ o[:, r]
        lse[r] = L
    return out, lse
