"""GPU parity with Q8_0 values (kvattn_geom.v_type = KVATTN_V_Q8_0, the
q8_0 / q8_0 cache pair of the Vulkan long-context page, section on the KV
cache types): the pages kvattn_quantize_pages writes equal the oracle's bit
for bit (bytes outside the written range untouched), decode and verify match
the oracle's attention within the decode bar (2e-3 max-abs), gather copies the
larger value records bit for bit, and chunked prefill matches the oracle
within the prefill bar (1e-2 max-abs)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from kvtest_util import DEV, Pools, compare, fill, gpu, host, prefill_checked

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3
PRE_TOL = 1e-2
V8 = kv.V_Q8_0


@pytest.mark.parametrize("pos0,n_tok", [(0, 128), (0, 300), (5, 1), (37, 90), (120, 20),
                                        (64, 32), (250, 517)])
def test_quantize_q8_values_bitexact(pos0, n_tok):
    n_kv, n_phys = 3, 12
    g = np.random.default_rng(pos0 * 1000 + n_tok)
    n_logical = (pos0 + n_tok + 127) // 128 + 1
    table = g.permutation(n_phys)[:n_logical].astype(np.int32)
    pools = Pools(n_phys, n_kv, 6, init_seed=pos0 + 1, v_type=V8)
    K = g.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    V = (g.standard_normal((n_tok, n_kv, 256)) * np.exp(g.standard_normal((n_tok, n_kv, 1)))
         ).astype(np.float32)
    V[0, 0, :32] = 0.0                       # zero block: codes 0, scale +0
    V[-1, -1, 32:64] = 1e-8                  # scale underflows to 0 in binary16
    V[0, -1, 64:96] = 127.0 * 3.0            # exact multiples of the scale
    pools.write(K, V, pos0, table)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all(), "K bytes differ"
    assert (gv == pools.ov).all(), "V bytes differ"


@pytest.mark.parametrize("n_kv,gqa,n_q_tok,kv_len,n_splits", [
    (4, 6, 1, 5000, 0),           # decode, one query row tile
    (2, 6, 4, 3000, 0),           # verify: 24 rows, two row tiles
    (1, 8, 4, 130, 0),            # a page and two tokens
    (2, 6, 4, 64 * 128 + 77, 7),  # chosen split count, ragged last page
    (1, 1, 1, 1, 0),              # one key
])
def test_decode_q8_values_matches_oracle(n_kv, gqa, n_q_tok, kv_len, n_splits):
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=kv_len + n_q_tok, init_seed=3, v_type=V8)
    g = np.random.default_rng(kv_len)
    q = g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32)
    n_pages = (kv_len + 127) // 128
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, n_splits=n_splits)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def test_sparse_decode_q8_values_matches_oracle():
    n_kv, gqa, kv_len = 2, 6, 40 * 128 + 9
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=11, init_seed=4, v_type=V8)
    g = np.random.default_rng(12)
    n_pages = (kv_len + 127) // 128
    blocks = np.stack([np.r_[np.sort(g.choice(n_pages - 1, 9, replace=False)), n_pages - 1]
                       for _ in range(n_kv)]).astype(np.int32)
    q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, blocks=gpu(blocks, torch.int32))
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                 blocks=blocks)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def test_q8_values_are_closer_to_exact_attention():
    """The same tokens cached with Q8_0 values give attention closer to the
    unquantised result than with Q4_0 values (keys identical in both)."""
    n_kv, gqa, kv_len = 1, 6, 2000
    res = {}
    for vt in (kv.V_Q4_0, V8):
        pools, table, K, V = fill(n_kv, gqa, kv_len, seed=21, v_type=vt)
        q = np.random.default_rng(22).standard_normal((1, gqa, 256)).astype(np.float32)
        out, _ = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv,
                                  gpu(table, torch.int32), kv_len, 1 / 16)
        res[vt] = host(out)
    o, _ = oracle.attend_rows(q.reshape(-1, 256), K[:, 0].astype(np.float64),
                              V[:, 0].astype(np.float64), np.arange(kv_len),
                              np.full(gqa, kv_len - 1), 1 / 16)
    e4 = np.abs(res[kv.V_Q4_0].reshape(-1, 256) - o).max()
    e8 = np.abs(res[V8].reshape(-1, 256) - o).max()
    assert e8 < e4 / 4, (e8, e4)


def test_gather_q8_values_bitexact():
    n_kv, n_phys, n_sel = 2, 10, 5
    g = np.random.default_rng(31)
    pools = Pools(n_phys, n_kv, 6, init_seed=8, v_type=V8)
    table = g.permutation(n_phys).astype(np.int32)
    blocks = np.stack([g.permutation(n_phys)[:n_sel] for _ in range(n_kv)]).astype(np.int32)
    dk = torch.zeros(n_sel * n_kv * quant.K_RECORD_BYTES, dtype=torch.uint8, device=DEV)
    dv = torch.zeros(n_sel * n_kv * quant.V8_RECORD_BYTES, dtype=torch.uint8, device=DEV)
    db = kv.kvattn_gather_blocks(pools.geom, pools.gk, pools.gv, gpu(table, torch.int32),
                                 gpu(blocks, torch.int32), n_sel, dk, dv)
    torch.cuda.synchronize()
    got_k = host(dk).reshape(n_sel, n_kv, -1)
    got_v = host(dv).reshape(n_sel, n_kv, -1)
    assert (host(db) == np.arange(n_sel)).all()
    for h in range(n_kv):
        for i in range(n_sel):
            assert (got_k[i, h] == pools.ok[table[blocks[h, i]], h]).all()
            assert (got_v[i, h] == pools.ov[table[blocks[h, i]], h]).all()


@pytest.mark.parametrize("chunk,pos0,gqa,n_kv,n_groups", [
    (128, 0, 6, 1, 0),         # first chunk: causal inside one page
    (200, 1000, 3, 2, 0),      # ragged chunk and history, several groups
    (512, 64 * 128, 6, 1, 5),  # a 512-token chunk after 64 pages, chosen group count
    (1, 5, 1, 1, 0),           # one query row, six keys
])
def test_prefill_q8_values_matches_oracle(chunk, pos0, gqa, n_kv, n_groups):
    kv_len = pos0 + chunk
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=chunk + pos0, init_seed=8, v_type=V8)
    q = np.random.default_rng(kv_len).standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
    out, lse = prefill_checked(pools.geom, gpu(q), pools.gk, pools.gv,
                                       gpu(table, torch.int32), pos0, 1 / 16, n_groups=n_groups)
    ref_o, ref_l = oracle.prefill_chunk(q, gqa, pools.ok, pools.ov, table, len(table), pos0,
                                        1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= PRE_TOL, eo
    assert el <= 5e-3 and rr <= 5e-3, (el, rr)
