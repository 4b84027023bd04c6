"""Seeded synthetic inputs for the five workloads, shared by the tests, the
benchmark and the CPU oracle runs. Holds no step of the attention method:
only random draws, shapes and the needle construction of the selection
workload.

Every draw comes from numpy's PCG64 seeded with
SeedSequence([seed, config, layer, head, role]), so any (layer, head) slice can
be regenerated on its own, on any host, bit for bit.

Shapes follow the pages: 16 full-attention layers x 4 KV heads x head_dim 256
([VULKAN] "模型結構"), grouped-query factor 6 (24 query heads), 128-token
pages ([KVMEM] --kvmem-block-tokens 128), prefill micro-batch 512 ([STREAM]
step ④ -ub 512), budget 32768 = 256 blocks plus a 16384-token (128-block)
reserve ([KVMEM] 測試口徑), 20 needles ([KVMEM] "Recall 測試"), verify batches
of 1 + 3 drafts ([RDNA4] verify batches). The pages' prompts (SQLite source,
needle-in-a-haystack text) are not reproduced; N(0,1) data of the same shapes
stands in for them.
"""
import concurrent.futures as _cf
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 256
PAGE_TOKENS = 128

ROLE_K, ROLE_V, ROLE_Q, ROLE_OUTLIER, ROLE_PAGES, ROLE_NEEDLE, ROLE_FAINT = range(7)


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    n_layers: int
    n_kv: int
    gqa: int
    kv_len: int          # tokens in the cache, including decode/verify queries
    n_q_tok: int         # decode / verify query tokens (0 for prefill)
    chunk: int = 0       # prefill chunk (its tokens are part of kv_len)
    outliers: int = 0    # outlier channels per (layer, KV head), x8 magnitude
    permuted: bool = True
    k_top: int = 0       # selection: top-k blocks outside the recent window
    n_recent: int = 0    # selection: recent blocks always kept
    n_needles: int = 0
    seed: int = 0

    @property
    def n_heads(self):
        return self.n_kv * self.gqa

    @property
    def n_pages(self):
        return (self.kv_len + PAGE_TOKENS - 1) // PAGE_TOKENS

    @property
    def pos0(self):
        """First position of the prefill chunk."""
        return self.kv_len - self.chunk


WORKLOADS = {
    1: Workload(1, "tiny-decode-4k", 1, 1, 6, 4096, 1, permuted=False),
    2: Workload(2, "decode-131k", 16, 4, 6, 131072, 1, outliers=4),
    3: Workload(3, "verify-262k", 16, 4, 6, 262144, 4),
    4: Workload(4, "prefill-512-after-262k", 16, 4, 6, 262144 + 512, 0, chunk=512),
    5: Workload(5, "kvmem-523k", 16, 4, 6, 523264, 1, k_top=256, n_recent=128,
                n_needles=20),
}


def rng(w, layer, head, role):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([w.seed, w.idx, layer, head, role])))


def normal(gen, shape):
    out = np.empty(shape, np.float32)
    gen.standard_normal(dtype=np.float32, out=out)
    return out


def page_table(w):
    """Logical -> physical page map: identity, or one seeded permutation shared
    by all layers and heads."""
    if not w.permuted:
        return np.arange(w.n_pages, dtype=np.int32)
    return rng(w, 0, 0, ROLE_PAGES).permutation(w.n_pages).astype(np.int32)


def queries(w, layer):
    """float32 [n_q_tok or chunk, n_heads, 256], N(0,1)."""
    n = w.chunk if w.chunk else w.n_q_tok
    return normal(rng(w, layer, 0, ROLE_Q), (n, w.n_heads, HEAD_DIM))


def outlier_channels(w, layer, head):
    return rng(w, layer, head, ROLE_OUTLIER).choice(HEAD_DIM, w.outliers, replace=False)


def needle_blocks(w):
    """Distinct candidate blocks (outside the recent window) holding needles;
    the same blocks for every layer and head."""
    n_cand = w.n_pages - w.n_recent
    return np.sort(rng(w, 0, 0, ROLE_NEEDLE).choice(n_cand, w.n_needles, replace=False))


def _needle_keys(k, qgroup):
    """Turn keys toward the group's summed query: k' = |k| (u/2 + (sqrt3/2) w),
    u = unit(sum of the group's query vectors), w = unit(k - (k.u) u); the
    cosine between k' and u is exactly 1/2 before rounding to float32."""
    u = np.asarray(qgroup, np.float64).sum(axis=0)
    u /= np.linalg.norm(u)
    k64 = k.astype(np.float64)
    perp = k64 - (k64 @ u)[:, None] * u[None, :]
    perp /= np.linalg.norm(perp, axis=1, keepdims=True)
    nk = np.linalg.norm(k64, axis=1, keepdims=True)
    return (nk * (0.5 * u[None, :] + (np.sqrt(3.0) / 2.0) * perp)).astype(np.float32)


def kv_head(w, layer, head, q=None):
    """(K, V) float32 [kv_len, 256] for one (layer, KV head). For the selection
    workload `q` (that layer's queries) is needed to build the needles."""
    K = normal(rng(w, layer, head, ROLE_K), (w.kv_len, HEAD_DIM))
    V = normal(rng(w, layer, head, ROLE_V), (w.kv_len, HEAD_DIM))
    if w.outliers:
        ch = outlier_channels(w, layer, head)
        K[:, ch] *= np.float32(8.0)
        V[:, ch] *= np.float32(8.0)
    if w.n_needles:
        if q is None:
            q = queries(w, layer)
        grp = q[-1, head * w.gqa:(head + 1) * w.gqa]
        for b in needle_blocks(w):
            sl = slice(b * PAGE_TOKENS, (b + 1) * PAGE_TOKENS)
            K[sl] = _needle_keys(K[sl], grp)
    return K, V


def faint_needle_keys(w, layer, head, q, span_blocks, per_block=3):
    """Keys float32 [kv_len, 256] of one (layer, KV head) for the recall curve:
    N(0,1) keys in which each of w.n_needles blocks, drawn among the first
    span_blocks, holds `per_block` needle tokens (seeded slots) turned toward
    the group's summed query at cosine 1/2, the rest of the block plain.
    A block summary averages its 128 keys, so one faint fact in a block of
    noise moves it only a little above the noise: whether it ranks among the
    kept blocks depends on how many candidates compete, i.e. on the context
    length and the budget. The needles are mutually similar (all point at the
    same query direction), as in [KVMEM] "Recall 測試", where a miss returns
    another, similar needle."""
    K = normal(rng(w, layer, head, ROLE_K), (w.kv_len, HEAD_DIM))
    g = rng(w, layer, head, ROLE_FAINT)
    blocks = np.sort(rng(w, 0, 0, ROLE_FAINT).choice(span_blocks, w.n_needles, replace=False))
    grp = q[-1, head * w.gqa:(head + 1) * w.gqa]
    for b in blocks:
        slots = b * PAGE_TOKENS + g.choice(PAGE_TOKENS, per_block, replace=False)
        K[slots] = _needle_keys(K[slots], grp)
    return K, blocks


def kv_layer(w, layer, q=None, threads=8):
    """(K, V) float32 [kv_len, n_kv, 256] for one layer, heads drawn in parallel
    threads (numpy releases the GIL while drawing)."""
    K = np.empty((w.kv_len, w.n_kv, HEAD_DIM), np.float32)
    V = np.empty_like(K)

    def one(h):
        kh, vh = kv_head(w, layer, h, q)
        K[:, h] = kh
        V[:, h] = vh

    with _cf.ThreadPoolExecutor(min(threads, w.n_kv)) as ex:
        list(ex.map(one, range(w.n_kv)))
    return K, V


def small_case(seed, n_tok, n_kv, n_q, gqa, scale_kv=1.0):
    """Generic seeded small inputs: (K, V) [n_tok, n_kv, 256] and Q [n_q, n_kv*gqa, 256]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    K = (normal(g, (n_tok, n_kv, HEAD_DIM)) * np.float32(scale_kv)).astype(np.float32)
    V = (normal(g, (n_tok, n_kv, HEAD_DIM)) * np.float32(scale_kv)).astype(np.float32)
    Q = normal(g, (n_q, n_kv * gqa, HEAD_DIM))
    return K, V, Q
