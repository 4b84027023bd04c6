"""Oracle: KVMem-style block scoring and budgeted top-k selection.
Test infrastructure only (see the package docstring).

[KVMEM] 測試口徑: --kvmem-budget 32768 with --kvmem-block-tokens 128 keeps
budget/128 = 256 history blocks, plus --kvmem-gen-reserve 16384 for the recent
window; "Recall 測試": at budget 32768, 256 of 485 blocks stay on the GPU
(53% coverage); "Full-KV 對照": attention then runs over the ~48K-token
working set only. The pages do not say how blocks are scored; this build reads
it as (summed group query) . (block mean key), top-k outside the recent window
(so the working set is budget + reserve = 48K tokens), ties to the lowest
block index.
"""
import heapq

import numpy as np


def query_sum(q, gqa):
    """q_sel[h] = RN32(binary64 sum over the group's query heads, ascending g).
    q: float32 [n_kv*gqa, 256] -> float32 [n_kv, 256]."""
    q = np.asarray(q, np.float32).astype(np.float64)
    n_heads, D = q.shape
    n_kv = n_heads // gqa
    grouped = q.reshape(n_kv, gqa, D)                  # query head h*gqa + g
    acc = np.zeros((n_kv, D), np.float64)
    for g in range(gqa):                                # ascending g
        acc = acc + grouped[:, g]
    return acc.astype(np.float32)


def block_scores(q_sel, summaries):
    """score[b] = binary64 sum over dims n = 0..255 in ascending order of
    q_sel[n] * summary[b][n]. Each product of two binary32 values is exact in
    binary64, so only the summation order matters, and it is fixed.
    q_sel float32 [256]; summaries float32 [NB, 256] -> float64 [NB]."""
    q = np.asarray(q_sel, np.float32).astype(np.float64)
    s = np.asarray(summaries, np.float32).astype(np.float64)
    acc = np.zeros(s.shape[0], np.float64)
    for n in range(s.shape[1]):                         # ascending n
        acc = acc + q[n] * s[:, n]
    return acc


def select_count(n_blocks, n_recent, k_top):
    """Blocks kept per head: min(k_top, NB - R) + R with R = min(n_recent, NB)."""
    r = min(n_recent, n_blocks)
    return min(k_top, n_blocks - r) + r


def select_blocks(scores, n_blocks, n_recent, k_top, method="sort"):
    """Ascending list of kept blocks for one head: the top min(k_top, NB-R)
    candidates b in [0, NB-R) by (score descending, b ascending), together with
    the recent blocks NB-R .. NB-1. -0 and +0 rank equal (Python compares them
    equal). `method` picks one of two independent brute-force orderings
    ("sort": full sort; "heap": heapq.nsmallest) so tests can cross-check."""
    r = min(n_recent, n_blocks)
    n_cand = n_blocks - r
    k = min(k_top, n_cand)
    sc = [float(x) for x in np.asarray(scores, np.float64)[:n_cand]]
    key = lambda b: (-sc[b], b)                          # noqa: E731
    if method == "sort":
        top = sorted(range(n_cand), key=key)[:k]
    elif method == "heap":
        top = heapq.nsmallest(k, range(n_cand), key=key)
    else:
        raise ValueError(method)
    return np.array(sorted(top) + list(range(n_cand, n_blocks)), np.int32)
