"""GPU parity of the fused append + decode (kvattn_append_decode).

Per case, on pools pre-filled with random bytes and a permuted page table:
 - the pool bytes it writes equal the oracle's quantisation of the new tokens
   bit for bit (and every other byte is untouched);
 - its out and lse equal kvattn_quantize_pages followed by kvattn_decode bit
   for bit, and the oracle's attention over the oracle's pool within the
   decode bar (2e-3 max-abs);
 - every key / value type pair: Q8_0, Q4_0 or Q5_1 keys (whole words per token),
   Q4_0 values (read-modify-write of shared words) or Q8_0 values (bytes);
 - with a summary array, the summary of a page the append completes equals
   the two-call path's and the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from kvtest_util import DEV, Pools, compare, gpu, host

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3

CASES = [
    # n_kv, gqa, n_q_tok, n_new, kv_len, n_splits, sparse
    (2, 6, 4, 4, 3 * 128 + 100, 0, False),     # verify: four tokens inside one group
    (2, 6, 4, 4, 2 * 128 + 34, 0, False),      # the new tokens straddle a group boundary
    (1, 6, 4, 4, 3 * 128 + 2, 0, False),       # ... and a page boundary
    (4, 6, 1, 1, 5000, 0, False),              # decode: one token
    (2, 3, 1, 32, 5 * 128 - 64, 0, False),     # one whole group: every word is new
    (2, 3, 2, 32, 5 * 128 - 50, 3, False),     # 32 tokens over two groups
    (1, 8, 3, 7, 1000, 0, False),              # an odd count
    (1, 6, 4, 4, 40, 1, False),                # the appended tile is a wave's first tile
    (2, 6, 4, 4, 9 * 128 + 3, 10, False),      # one page per split
    # one split over 193 pages: the appended tile is unit 120 of waves 0-3,
    # found after the search reloads the 64-unit page window
    (2, 6, 4, 4, 64 * 128 * 3 + 5, 1, False),
    (2, 6, 1, 3, 4 * 128, 0, True),            # sparse; completes a page (summary)
    (1, 6, 2, 2, 6 * 128 + 1, 0, True),        # sparse; the new tokens straddle two listed pages
    (2, 6, 4, 4, 3 * 128, 0, False),           # dense; completes the last page (summary)
    (1, 6, 1, 3, 5 * 128 + 1, 1, False),       # dense, one split; completes the next-to-last page
    (2, 6, 4, 4, 40 * 128, 7, False),          # dense, seven splits; completes the last page
    # dense, two splits of two pages: the completed page 2 is the first unit
    # of split 1, streamed by waves 4-7; the new tokens straddle into page 3
    (1, 6, 1, 3, 3 * 128 + 1, 2, False),
]


def plant_edges(Kn, Vn):
    """Quantiser edge rules inside the appended tokens."""
    Kn[0, 0, :32] = 0.0                                  # zero block
    Vn[0, 0, 32:64] = 0.0
    Vn[0, 0, 32 + 3], Vn[0, 0, 32 + 7] = 1.0, -1.0       # tie across lanes: lowest index
    Vn[0, 0, 64:96] = 0.25
    Vn[0, 0, 64 + 30], Vn[0, 0, 64 + 9] = 3.0, -3.0      # tie, far apart
    Vn[0, 0, 96 + 5], Vn[0, 0, 96 + 6] = -4.5, 4.5       # tie inside one group of four
    Kn[0, 0, 128:160] *= 4.0                             # outlier block (the logits stay moderate)


@pytest.mark.parametrize("k_type,v_type", [(kv.K_Q8_0, kv.V_Q4_0), (kv.K_Q8_0, kv.V_Q8_0),
                                            (kv.K_Q4_0, kv.V_Q4_0), (kv.K_Q4_0, kv.V_Q8_0),
                                            (kv.K_Q5_1, kv.V_Q4_0)])
@pytest.mark.parametrize("n_kv,gqa,n_q_tok,n_new,kv_len,n_splits,sparse", CASES)
def test_append_decode_matches_quantize_then_decode(n_kv, gqa, n_q_tok, n_new, kv_len, n_splits,
                                                    sparse, k_type, v_type):
    g = np.random.default_rng(kv_len * 7 + n_new)
    n_pages = (kv_len + 127) // 128
    n_phys = n_pages + 3
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    pos0 = kv_len - n_new
    pools = Pools(n_phys, n_kv, gqa, init_seed=kv_len, v_type=v_type, k_type=k_type)
    if pos0 > 0:
        Kh = g.standard_normal((pos0, n_kv, 256)).astype(np.float32)
        Vh = g.standard_normal((pos0, n_kv, 256)).astype(np.float32)
        pools.write(Kh, Vh, 0, table)
    Kn = g.standard_normal((n_new, n_kv, 256)).astype(np.float32)
    Vn = g.standard_normal((n_new, n_kv, 256)).astype(np.float32)
    plant_edges(Kn, Vn)
    q = g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32)
    blocks = None
    if sparse:
        new_pages = sorted({p // 128 for p in range(pos0, kv_len)})
        rows = []
        for h in range(n_kv):
            rest = [p for p in range(n_pages) if p not in new_pages]
            pick = sorted(g.choice(rest, 2, replace=False).tolist()) if len(rest) >= 2 else rest
            rows.append(sorted(pick + new_pages))
        blocks = np.array(rows, np.int32)
    table_d = gpu(table, torch.int32)
    blocks_d = None if blocks is None else gpu(blocks, torch.int32)

    # the two-call path on a copy of the device pools
    gk2, gv2 = pools.gk.clone(), pools.gv.clone()
    summ = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    summ2 = summ.clone()
    kv.kvattn_quantize_pages(pools.geom, gpu(Kn), gpu(Vn), pos0, table_d, gk2, gv2, summ2)
    o2, l2 = kv.kvattn_decode(pools.geom, gpu(q), gk2, gv2, table_d, kv_len, 1 / 16,
                              blocks=blocks_d, n_splits=n_splits)
    # the fused path
    out, lse = kv.kvattn_append_decode(pools.geom, gpu(Kn), gpu(Vn), gpu(q), pools.gk, pools.gv,
                                       table_d, kv_len, 1 / 16, blocks=blocks_d, k_summary=summ,
                                       n_splits=n_splits)
    torch.cuda.synchronize()

    quant.quantize_into_pool(Kn, Vn, pos0, table, pools.ok, pools.ov)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all(), "K bytes differ from the oracle"
    assert (gv == pools.ov).all(), "V bytes differ from the oracle"
    assert torch.equal(pools.gk, gk2) and torch.equal(pools.gv, gv2)
    assert torch.equal(out, o2) and torch.equal(lse, l2), "fused result differs from two calls"

    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                 blocks=blocks)
    eo, el, rr = compare(out, lse, ref_o.reshape(n_q_tok, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)

    # the summary of a page the append completes (written by the decode
    # launch) equals the separate summary launch's and the oracle's
    assert torch.equal(summ, summ2)
    full = kv_len // 128
    done = [p for p in range(pos0 // 128, full)]
    ref_s = quant.summaries_from_pool(pools.ok, table, full, n_kv)
    got = host(summ)
    for p in range(n_pages):
        if p in done:
            assert (got[:, p].view(np.uint32) == ref_s[:, p].view(np.uint32)).all()
        else:
            assert (got[:, p] == 0).all()


def test_append_decode_repeated_steps():
    """A decode loop: each step appends one token and attends; after 40 steps
    (crossing a page boundary) the pool equals the oracle's bit for bit."""
    n_kv, gqa, n_phys = 2, 6, 6
    g = np.random.default_rng(77)
    table = g.permutation(n_phys)[:4].astype(np.int32)
    start = 120
    pools = Pools(n_phys, n_kv, gqa, init_seed=78)
    Kh = g.standard_normal((start, n_kv, 256)).astype(np.float32)
    Vh = g.standard_normal((start, n_kv, 256)).astype(np.float32)
    pools.write(Kh, Vh, 0, table)
    table_d = gpu(table, torch.int32)
    for step in range(40):
        kv_len = start + step + 1
        Kn = g.standard_normal((1, n_kv, 256)).astype(np.float32)
        Vn = g.standard_normal((1, n_kv, 256)).astype(np.float32)
        q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
        out, lse = kv.kvattn_append_decode(pools.geom, gpu(Kn), gpu(Vn), gpu(q), pools.gk,
                                           pools.gv, table_d, kv_len, 1 / 16)
        quant.quantize_into_pool(Kn, Vn, kv_len - 1, table, pools.ok, pools.ov)
        if step % 13 == 0 or step == 39:
            ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, len(table), kv_len,
                                         1 / 16)
            eo, el, rr = compare(out, lse, ref_o, ref_l)
            assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (step, eo, el, rr)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all() and (gv == pools.ov).all()


def test_append_summary_of_large_q8_keys():
    """Q8_0 keys of magnitude 5e6 .. 8e6 (scales near the binary16 limit): the
    magnitudes of a page add up past 2^53 units of 2^-24, so the summary takes
    the ascending binary64 sum as written; it still equals the separate
    summary launch and the oracle bit for bit (attention over such keys is
    outside the decode's range and is not checked). Q4_0 and Q5_1 keys cannot
    reach that bound."""
    n_kv, gqa, kv_len, n_new = 1, 6, 2 * 128, 2
    g = np.random.default_rng(90)
    n_pages = kv_len // 128
    table = np.array([2, 0], np.int32)
    pools = Pools(3, n_kv, gqa, init_seed=91, k_type=kv.K_Q8_0)
    pos0 = kv_len - n_new

    def big(n):
        mag = g.uniform(5.0e6, 8.0e6, (n, n_kv, 256))
        return (mag * g.choice([-1.0, 1.0], mag.shape)).astype(np.float32)

    pools.write(big(pos0), g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
    Kn = big(n_new)
    Vn = g.standard_normal((n_new, n_kv, 256)).astype(np.float32)
    q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    table_d = gpu(table, torch.int32)
    gk2, gv2 = pools.gk.clone(), pools.gv.clone()
    summ = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    summ2 = summ.clone()
    kv.kvattn_quantize_pages(pools.geom, gpu(Kn), gpu(Vn), pos0, table_d, gk2, gv2, summ2)
    kv.kvattn_append_decode(pools.geom, gpu(Kn), gpu(Vn), gpu(q), pools.gk, pools.gv, table_d,
                            kv_len, 1 / 16, k_summary=summ)
    torch.cuda.synchronize()
    quant.quantize_into_pool(Kn, Vn, pos0, table, pools.ok, pools.ov)
    ref_s = quant.summaries_from_pool(pools.ok, table, n_pages, n_kv)
    kh = quant.dequantize_keys(pools.ok[table[1]])
    assert np.isfinite(kh).all()
    assert np.abs(kh).sum(axis=-2).max() * 2.0 ** 24 >= 2.0 ** 53  # the fallback is taken
    assert torch.equal(summ[:, 1], summ2[:, 1])
    assert (host(summ)[:, 1].view(np.uint32) == ref_s[:, 1].view(np.uint32)).all()


@pytest.mark.parametrize("k_type,sparse,n_new,kv_len,n_splits", [
    (kv.K_Q8_0, False, 4, 3 * 128 + 2, 5),     # the new tokens complete page 2
    (kv.K_Q4_0, True, 1, 7 * 128, 3),          # sparse list; the append completes page 6
    (kv.K_Q5_1, False, 32, 6 * 128 - 50, 4),   # 32 new tokens; uneven splits of six pages
])
def test_append_decode_partials_merge_to_append_decode(k_type, sparse, n_new, kv_len, n_splits):
    """kvattn_append_decode_partials writes the bytes and summaries
    kvattn_append_decode writes, and kvattn_merge_lse of its partials is
    kvattn_append_decode's result at the same split count, bit for bit."""
    n_kv, gqa, n_q_tok = 2, 6, 2
    g = np.random.default_rng(kv_len + n_new)
    n_pages = (kv_len + 127) // 128
    table = g.permutation(n_pages + 2)[:n_pages].astype(np.int32)
    pools = Pools(n_pages + 2, n_kv, gqa, init_seed=kv_len, k_type=k_type)
    pos0 = kv_len - n_new
    pools.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
    Kn = gpu(g.standard_normal((n_new, n_kv, 256)).astype(np.float32))
    Vn = gpu(g.standard_normal((n_new, n_kv, 256)).astype(np.float32))
    q = gpu(g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32))
    blocks = None
    if sparse:
        rows = [sorted(set(g.choice(n_pages - 1, 3, replace=False).tolist()) | {n_pages - 1})
                for _ in range(n_kv)]
        blocks = gpu(np.array(rows, np.int32), torch.int32)
    table_d = gpu(table, torch.int32)
    gk2, gv2 = pools.gk.clone(), pools.gv.clone()
    summ = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    summ2 = summ.clone()
    o_part, l_part = kv.kvattn_append_decode_partials(pools.geom, Kn, Vn, q, pools.gk, pools.gv,
                                                      table_d, kv_len, 1 / 16, n_splits,
                                                      blocks=blocks, k_summary=summ)
    rows_n = n_q_tok * n_kv * gqa
    out, lse = kv.kvattn_merge_lse(o_part, l_part)
    o2, l2 = kv.kvattn_append_decode(pools.geom, Kn, Vn, q, gk2, gv2, table_d, kv_len, 1 / 16,
                                     blocks=blocks, k_summary=summ2, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(pools.gk, gk2) and torch.equal(pools.gv, gv2)
    assert torch.equal(summ, summ2)
    assert torch.equal(out, o2.view(rows_n, 256)) and torch.equal(lse, l2.view(rows_n))
