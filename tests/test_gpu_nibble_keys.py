"""GPU parity with nibble keys: Q4_0 (kvattn_geom.k_type = KVATTN_K_Q4_0: the
q4_0/q4_0 pair, 18 KiB per token for K + V at 16 layers x 4 KV heads, the
Vulkan long-context page's 坑 2) and Q5_1 (KVATTN_K_Q5_1: the q5_1/q4_0 pair
of that page's 坑 3), each also with Q8_0 values: the pages
and block summaries kvattn_quantize_pages writes equal the oracle's bit for
bit, block selection over those summaries equals the oracle's, decode, verify
and chunked prefill match the oracle's attention within their bars (2e-3 /
1e-2 max-abs), and gather copies the smaller key records bit for bit."""
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
KTYPES = [kv.K_Q4_0, kv.K_Q5_1]


@pytest.mark.parametrize("k_type", KTYPES)
@pytest.mark.parametrize("v_type", [kv.V_Q4_0, kv.V_Q8_0])
@pytest.mark.parametrize("pos0,n_tok", [(0, 256), (5, 1), (37, 90), (120, 20), (250, 517)])
def test_quantize_nibble_keys_bitexact_with_summaries(pos0, n_tok, v_type, k_type):
    n_kv, n_phys = 3, 12
    g = np.random.default_rng(pos0 * 1000 + n_tok + v_type + 7 * k_type)
    n_logical = (pos0 + n_tok + 127) // 128 + 1
    table = g.permutation(n_phys)[:n_logical].astype(np.int32)
    pools = Pools(n_phys, n_kv, 6, init_seed=pos0 + 1, v_type=v_type, k_type=k_type)
    K = (g.standard_normal((n_tok, n_kv, 256)) * np.exp(g.standard_normal((n_tok, n_kv, 1)))
         ).astype(np.float32)
    V = g.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    K[0, 0, :32] = 0.0                       # zero block: scale +0
    K[0, 1, :32] = -0.75                     # constant block (Q5_1: d = 0, every code 0)
    K[-1, -1, 32:64] = 0.25
    K[-1, -1, 40], K[-1, -1, 60] = 3.0, -3.0  # tie: the lower index sets the sign
    K[0, -1, 64:96] = 1e-9                   # scale underflows in binary16
    summ = torch.zeros((n_kv, n_logical, 256), dtype=torch.float32, device=DEV)
    pools.write(K, V, pos0, table, summ)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all(), "K bytes differ"
    assert (gv == pools.ov).all(), "V bytes differ"
    full = [p for p in range(pos0 // 128, (pos0 + n_tok) // 128)]
    ref = quant.summaries_from_pool(pools.ok, table, n_logical, n_kv)
    got = host(summ)
    for p in range(n_logical):
        if p in full:
            # slots before pos0 hold the random initial bytes, whose scales can be
            # inf or NaN: a NaN sum matches as NaN (payloads differ), all else bitwise
            nan = np.isnan(ref[:, p])
            assert (np.isnan(got[:, p]) == nan).all(), p
            assert (got[:, p][~nan].view(np.uint32) == ref[:, p][~nan].view(np.uint32)).all(), p
        else:
            assert (got[:, p] == 0).all()


@pytest.mark.parametrize("k_type", KTYPES)
@pytest.mark.parametrize("v_type", [kv.V_Q4_0, kv.V_Q8_0])
@pytest.mark.parametrize("n_kv,gqa,n_q_tok,kv_len,n_splits", [
    (4, 6, 1, 5000, 0),           # decode, one query row tile
    (2, 6, 4, 3000, 0),           # verify: 24 rows, two row tiles
    (1, 8, 4, 130, 0),            # a page and two tokens
    (2, 6, 4, 64 * 128 + 77, 7),  # chosen split count, ragged last page
    (1, 1, 1, 1, 0),              # one key
])
def test_decode_nibble_keys_matches_oracle(n_kv, gqa, n_q_tok, kv_len, n_splits, v_type, k_type):
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=kv_len + n_q_tok, init_seed=3, v_type=v_type,
                              k_type=k_type)
    g = np.random.default_rng(kv_len)
    q = g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32)
    n_pages = (kv_len + 127) // 128
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, n_splits=n_splits)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


@pytest.mark.parametrize("k_type", KTYPES)
def test_select_and_sparse_decode_nibble_keys(k_type):
    """KVMem over a nibble-key cache: summaries, top-k selection and sparse
    decode over the kept blocks, each against the oracle."""
    n_kv, gqa, n_pages, n_recent, k_top = 2, 6, 40, 6, 9
    kv_len = n_pages * 128 - 17
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=41, init_seed=5, k_type=k_type)
    summ = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    g = np.random.default_rng(42)
    # rewrite the full pages with summaries (same bytes: quantisation is deterministic)
    K = g.standard_normal((kv_len, n_kv, 256)).astype(np.float32)
    V = g.standard_normal((kv_len, n_kv, 256)).astype(np.float32)
    pools.write(K, V, 0, table, summ)
    q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    blocks = kv.kvattn_select_blocks(pools.geom, gpu(q[0]), summ, n_pages, n_pages, n_recent,
                                     k_top)
    torch.cuda.synchronize()
    kept = host(blocks)
    qs = oracle.query_sum(q[0], gqa)
    summ_ref = quant.summaries_from_pool(pools.ok, table, n_pages - 1, n_kv)
    assert (host(summ)[:, :n_pages - 1].view(np.uint32) == summ_ref.view(np.uint32)).all()
    for h in range(n_kv):
        sc = oracle.block_scores(qs[h], summ_ref[h, :n_pages - n_recent])
        ref = oracle.select_blocks(np.r_[sc, np.zeros(n_recent)], n_pages, n_recent, k_top)
        assert (kept[h] == ref).all(), (h, kept[h], ref)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, blocks=blocks)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                 blocks=kept)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


@pytest.mark.parametrize("k_type", KTYPES)
@pytest.mark.parametrize("v_type", [kv.V_Q4_0, kv.V_Q8_0])
@pytest.mark.parametrize("chunk,pos0,gqa,n_kv,n_groups", [
    (128, 0, 6, 1, 0),         # first chunk: causal inside one page
    (200, 1000, 3, 2, 0),      # ragged chunk and history, several groups
    (512, 64 * 128, 6, 1, 5),  # a 512-token chunk after 64 pages, chosen group count
    (1, 5, 1, 1, 0),           # one query row, six keys
])
def test_prefill_nibble_keys_matches_oracle(chunk, pos0, gqa, n_kv, n_groups, v_type, k_type):
    kv_len = pos0 + chunk
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=chunk + pos0, init_seed=8, v_type=v_type,
                              k_type=k_type)
    q = np.random.default_rng(kv_len).standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
    out, lse = prefill_checked(pools.geom, gpu(q), pools.gk, pools.gv,
                                       gpu(table, torch.int32), pos0, 1 / 16, n_groups=n_groups)
    ref_o, ref_l = oracle.prefill_chunk(q, gqa, pools.ok, pools.ov, table, len(table), pos0,
                                        1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= PRE_TOL, eo
    assert el <= 5e-3 and rr <= 5e-3, (el, rr)


@pytest.mark.parametrize("k_type", KTYPES)
def test_gather_nibble_keys_bitexact(k_type):
    n_kv, n_phys, n_sel = 2, 10, 5
    g = np.random.default_rng(33)
    pools = Pools(n_phys, n_kv, 6, init_seed=8, k_type=k_type)
    table = g.permutation(n_phys).astype(np.int32)
    blocks = np.stack([g.permutation(n_phys)[:n_sel] for _ in range(n_kv)]).astype(np.int32)
    dk = torch.zeros(n_sel * n_kv * pools.geom.k_record_bytes, dtype=torch.uint8, device=DEV)
    dv = torch.zeros(n_sel * n_kv * quant.V_RECORD_BYTES, dtype=torch.uint8, device=DEV)
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
