"""GPU tests of kvattn_decode's split partials and their LSE merge.

 - the result equals kvattn_decode_partials + kvattn_merge_lse bit for bit,
   for one and four query tokens, one and four KV heads, 1 to 64 splits, and
   the oracle within the decode bar;
 - the workspace's counters are zero after every call;
 - ten back-to-back launches on one workspace, and a HIP graph replayed
   several times with eager work between replays, give identical bits;
 - more than 64 splits (another merge path) still match the oracle;
 - values up to the binary16 range stay finite and match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_paged_amd as kv
from kvtest_util import DEV, compare, fill, gpu, host

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3


def counters(ws):
    torch.cuda.synchronize()
    return host(ws[:kv.WORKSPACE_SYNC_BYTES].view(torch.int32))


@pytest.mark.parametrize("n_kv,gqa,n_q_tok,kv_len,n_splits", [
    (1, 6, 1, 4096, 0),
    (4, 6, 4, 5000, 0),
    (4, 6, 1, 9000, 64),
    (2, 6, 4, 3000, 1),
    (2, 8, 3, 2000, 7),
    (4, 6, 4, 64 * 128 + 77, 64),
    (1, 32, 1, 700, 5),
    # many KV heads with few rows each; 28 x 64 splits: more workgroups than
    # fit on the device at once
    (28, 1, 3, 600, 0),
    (28, 1, 4, 64 * 128 + 3, 64),
])
def test_decode_is_partials_plus_merge(n_kv, gqa, n_q_tok, kv_len, n_splits):
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=kv_len + n_kv, init_seed=3)
    g = np.random.default_rng(kv_len)
    q = gpu(g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32))
    td = gpu(table, torch.int32)
    ws = kv.workspace(64 << 20, DEV)
    out, lse = kv.kvattn_decode(pools.geom, q, pools.gk, pools.gv, td, kv_len, 1 / 16,
                                n_splits=n_splits, workspace=ws)
    S = n_splits or kv.kvattn_decode_splits(pools.geom, len(table))
    S = min(S, len(table))
    op, lp = kv.kvattn_decode_partials(pools.geom, q, pools.gk, pools.gv, td, kv_len, 1 / 16, S)
    o2, l2 = kv.kvattn_merge_lse(op, lp)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(-1, 256), o2.reshape(-1, 256))
    assert torch.equal(lse.reshape(-1), l2.reshape(-1))
    assert not counters(ws).any(), "counters not left zero"
    ref_o, ref_l = oracle.decode(host(q), gqa, pools.ok, pools.ov, table, len(table), kv_len,
                                 1 / 16)
    eo, el, rr = compare(out, lse, ref_o.reshape(n_q_tok, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def test_decode_repeated_launches_and_graph_replays():
    """Ten back-to-back launches on one workspace, then a graph of the call
    replayed five times with eager work between replays: identical bits."""
    n_kv, gqa, kv_len = 4, 6, 70 * 128 + 5
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=71, init_seed=4)
    q = gpu(np.random.default_rng(72).standard_normal((4, n_kv * gqa, 256)).astype(np.float32))
    td = gpu(table, torch.int32)
    ws = kv.workspace(64 << 20, DEV)
    outs = []
    for _ in range(10):
        o, l_ = kv.kvattn_decode(pools.geom, q, pools.gk, pools.gv, td, kv_len, 1 / 16,
                                 workspace=ws)
        outs.append((o, l_))
    torch.cuda.synchronize()
    for o, l_ in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l_, outs[0][1])
    assert not counters(ws).any()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kv.kvattn_decode(pools.geom, q, pools.gk, pools.gv, td, kv_len, 1 / 16, out=out, lse=lse,
                         workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kv.kvattn_decode(pools.geom, q, pools.gk, pools.gv, td, kv_len, 1 / 16, out=out, lse=lse,
                         workspace=ws)
    for _ in range(5):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, outs[0][0]) and torch.equal(lse, outs[0][1])
        assert not counters(ws).any()


def test_more_than_64_splits():
    n_kv, gqa, kv_len = 1, 6, 100 * 128
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=73)
    q = np.random.default_rng(74).standard_normal((2, gqa, 256)).astype(np.float32)
    ws = kv.workspace(64 << 20, DEV)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, n_splits=80, workspace=ws)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, len(table), kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o.reshape(2, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
    assert not counters(ws).any()


@pytest.mark.parametrize("v_type", [kv.V_Q4_0, kv.V_Q8_0])
@pytest.mark.parametrize("amax", [2500.0, 60000.0])
def test_decode_large_values_stay_finite(v_type, amax):
    """Values up to the binary16 range: the scaled probabilities P' * d_V are
    formed in f16, bounded by the rescale margin (P' <= 8) times the largest
    Q4_0 scale 65504 / 8. One block at amax, the rest N(0,1) * amax / 4."""
    n_kv, gqa, kv_len = 1, 6, 3000
    pools, table, K, V = fill(n_kv, gqa, kv_len, seed=77, v_type=v_type)
    g = np.random.default_rng(78)
    V2 = (g.standard_normal(V.shape) * (amax / 4)).astype(np.float32)
    V2 = np.clip(V2, -amax, amax)
    V2[1234, 0, 64:96] = 0.0
    V2[1234, 0, 70] = -amax                         # a block whose scale is amax / 8
    pools.write(K, V2, 0, table)
    q = g.standard_normal((4, gqa, 256)).astype(np.float32)
    q[:, :, :] *= 3.0                               # peaked softmax rows
    for n_splits in (0, 1):
        out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv,
                                    gpu(table, torch.int32), kv_len, 1 / 16, n_splits=n_splits)
        o = host(out)
        assert np.isfinite(o).all() and np.isfinite(host(lse)).all()
        ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, len(table), kv_len,
                                     1 / 16)
        eo, el, rr = compare(out, lse, ref_o.reshape(4, -1, 256), ref_l)
        assert eo <= DEC_TOL * amax and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
