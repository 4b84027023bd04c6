"""kvattn_append_decode_noalloc (the entry point that allocates nothing, its
split-K partials in the library's static per-GPU scratch) against
kvattn_append_decode with a workspace: out, lse, the pool bytes it writes and
the summary of a page the append completes, all bit for bit, over two calls
in a row on one GPU (the second smaller, so the scratch holds the first call's
larger partials), and a call whose partials exceed the scratch rejected before
anything is enqueued. Called through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_attention_paged_amd as kv
from kvtest_util import DEV, Pools, gpu

pytestmark = pytest.mark.gpu


def make_case(n_kv, gqa, n_q_tok, n_new, kv_len, seed, sparse=False):
    g = np.random.default_rng(seed)
    n_pages = (kv_len + 127) // 128
    n_phys = n_pages + 2
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    pos0 = kv_len - n_new
    pools = Pools(n_phys, n_kv, gqa, init_seed=seed + 1)
    pools.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
    k_new = gpu(g.standard_normal((n_new, n_kv, 256)).astype(np.float32))
    v_new = gpu(g.standard_normal((n_new, n_kv, 256)).astype(np.float32))
    q = gpu(g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32))
    blocks = None
    if sparse:
        new_pages = sorted({p // 128 for p in range(pos0, kv_len)})
        rows = []
        for _ in range(n_kv):
            rest = [p for p in range(n_pages) if p not in new_pages]
            rows.append(sorted(g.choice(rest, 5, replace=False).tolist() + new_pages))
        blocks = gpu(np.array(rows, np.int32))
    return pools, gpu(table), k_new, v_new, q, blocks, n_pages


def run_both(case, kv_len):
    pools, table, k_new, v_new, q, blocks, n_pages = case
    n_kv = pools.n_kv
    summ_ref = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    summ = summ_ref.clone()
    gk_ref, gv_ref = pools.gk.clone(), pools.gv.clone()
    o_ref, l_ref = kv.kvattn_append_decode(pools.geom, k_new, v_new, q, gk_ref, gv_ref, table,
                                           kv_len, 1 / 16, blocks=blocks, k_summary=summ_ref)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    kv.kvattn_append_decode_noalloc(pools.geom, k_new, v_new, q, pools.gk, pools.gv, table,
                                    kv_len, 1 / 16, out, lse, blocks=blocks, k_summary=summ)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref)
    assert torch.equal(lse, l_ref)
    assert torch.equal(pools.gk, gk_ref)
    assert torch.equal(pools.gv, gv_ref)
    assert torch.equal(summ, summ_ref)


def test_noalloc_matches_append_decode_twice_second_smaller():
    # verify: 4 query tokens x 4 KV heads x GQA 6 over 60 pages (96 rows,
    # 60 splits); the append completes page 59
    big = make_case(4, 6, 4, 4, 60 * 128, seed=11)
    print("noalloc: verify 4x4x6 over 60 pages", flush=True)
    run_both(big, 60 * 128)
    # decode: 1 token x 2 KV heads x GQA 3 over 9 pages with a ragged tail
    # (6 rows, 9 splits): fewer partials than the scratch still holds
    small = make_case(2, 3, 1, 1, 8 * 128 + 77, seed=12)
    print("noalloc: decode 1x2x3 over 9 pages", flush=True)
    run_both(small, 8 * 128 + 77)


def test_noalloc_sparse_after_dense():
    dense = make_case(2, 6, 2, 2, 30 * 128 + 5, seed=13)
    print("noalloc: dense 2x2x6 over 31 pages", flush=True)
    run_both(dense, 30 * 128 + 5)
    sparse = make_case(2, 6, 1, 3, 20 * 128, seed=14, sparse=True)
    print("noalloc: sparse 1x2x6, 6 listed pages", flush=True)
    run_both(sparse, 20 * 128)


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 8 KV heads x 32 rows at 64 splits: 64 * 256 * 1028 bytes > 16 MiB
    n_kv, gqa, n_q_tok, kv_len = 8, 8, 4, 64 * 128
    pools, table, k_new, v_new, q, _, _ = make_case(n_kv, gqa, n_q_tok, 1, kv_len, seed=15)
    out = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:2], dtype=torch.float32, device=DEV)
    gk0 = pools.gk.clone()
    with pytest.raises(kv.KvattnError) as e:
        kv.kvattn_append_decode_noalloc(pools.geom, k_new, v_new, q, pools.gk, pools.gv, table,
                                        kv_len, 1 / 16, out, lse, n_splits=64)
    assert e.value.code == 3  # KVATTN_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(pools.gk, gk0)          # nothing was enqueued
    assert not out.any()
    # the same shape at 32 splits fits and matches the workspace path
    o_ref, l_ref = kv.kvattn_append_decode(pools.geom, k_new, v_new, q, pools.gk.clone(),
                                           pools.gv.clone(), table, kv_len, 1 / 16, n_splits=32)
    kv.kvattn_append_decode_noalloc(pools.geom, k_new, v_new, q, pools.gk, pools.gv, table,
                                    kv_len, 1 / 16, out, lse, n_splits=32)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_replays_under_graph_capture():
    """The entry point's own use case: captured in a HIP graph (no allocation
    during capture) and replayed three times with eager work between the
    replays; every replay's out and lse equal the eager call's bit for bit
    (the append writes the same bytes each time)."""
    pools, table, k_new, v_new, q, blocks, n_pages = make_case(2, 6, 2, 2, 20 * 128 + 9, seed=16)
    kv_len = 20 * 128 + 9
    out0 = torch.empty_like(q)
    lse0 = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    kv.kvattn_append_decode_noalloc(pools.geom, k_new, v_new, q, pools.gk, pools.gv, table,
                                    kv_len, 1 / 16, out0, lse0)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kv.kvattn_append_decode_noalloc(pools.geom, k_new, v_new, q, pools.gk, pools.gv, table,
                                        kv_len, 1 / 16, out, lse, stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(lse, lse0), rep
        _ = (q * 2).sum().item()  # eager work between the replays
