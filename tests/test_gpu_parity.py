"""GPU parity: every entry point through the C ABI against the CPU oracle on the
same seeded inputs, at sizes that span several tiles and ragged tails.

Bars: page bytes, summaries and selected blocks bit-exact; decode max-abs
<= 2e-3 and prefill max-abs <= 1e-2 against binary64 attention over the
dequantised pages (the workload's stated tolerances), plus tighter internal
gates on relative RMS and lse, and exact closed forms for the structured
(indicator-page, peaked-key) cases.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from kvtest_util import DEV, Pools, compare, fill, gpu, host, prefill_checked

pytestmark = pytest.mark.gpu

DEC_TOL, PRE_TOL = 2e-3, 1e-2


def special_blocks(K, V):
    """Plant blocks that exercise the quantiser's edge rules."""
    K[0, 0, :32] = 0.0                                   # zero block
    V[0, 0, :32] = 0.0
    K[1, 0, 32:64] = 0.37                                # constant block
    V[1, 0, 32:64] = -2.5
    V[2, 0, 64:96] = 0.0
    V[2, 0, 64 + 3], V[2, 0, 64 + 7] = 1.0, -1.0         # magnitude tie: lowest index wins
    V[3, 0, 96:128] = 0.0
    V[3, 0, 96 + 5] = 1e-9                               # scale underflows in binary16
    K[4, 0, 128:160] *= 50.0                             # outlier block
    V[5, 0, :32] = ((np.arange(32) % 16 - 8) * 2.0 ** -5).astype(np.float32)  # exact grid
    V[6, 0, 160:192] = 0.25
    V[6, 0, 160 + 30], V[6, 0, 160 + 9], V[6, 0, 160 + 17] = 3.0, -3.0, 3.0  # tie over far-apart indices
    V[7, 0, 192:224] = -0.5
    V[7, 0, 192 + 1], V[7, 0, 192 + 2] = -4.0, 4.0       # tie inside one group of four


def test_quantize_bitexact_incremental():
    """Pool bytes after a sequence of appends (bulk, single token, ragged) on a
    permuted table, into pools pre-filled with random bytes, plus summaries."""
    n_kv, gqa, n_phys = 2, 6, 9
    g = np.random.default_rng(1)
    table = g.permutation(n_phys)[:6].astype(np.int32)
    total = 700
    K = g.standard_normal((total, n_kv, 256)).astype(np.float32)
    V = g.standard_normal((total, n_kv, 256)).astype(np.float32)
    special_blocks(K, V)
    pools = Pools(n_phys, n_kv, gqa, init_seed=2)
    summ = torch.zeros((n_kv, len(table), 256), dtype=torch.float32, device=DEV)
    for a, b in ((0, 200), (200, 201), (201, 256), (256, 641), (641, 700)):
        pools.write(K[a:b], V[a:b], a, table, summ)
        gk, gv = pools.gpu_bytes()
        assert (gk == pools.ok).all(), f"K bytes differ after writing [{a}, {b})"
        assert (gv == pools.ov).all(), f"V bytes differ after writing [{a}, {b})"
    full = total // 128
    ref = quant.summaries_from_pool(pools.ok, table, full, n_kv)
    got = host(summ)[:, :full]
    assert (got.view(np.uint32) == ref.view(np.uint32)).all()
    assert (host(summ)[:, full:] == 0).all()              # partial page: no summary


def test_quantize_skips_out_of_range_pages():
    n_kv, n_phys = 1, 3
    table = np.array([2, 7, 0], np.int32)                 # logical page 1 maps outside
    g = np.random.default_rng(3)
    K = g.standard_normal((384, n_kv, 256)).astype(np.float32)
    V = g.standard_normal((384, n_kv, 256)).astype(np.float32)
    pools = Pools(n_phys, n_kv, 1, init_seed=4)
    pools.write(K, V, 0, table)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all() and (gv == pools.ov).all()


def run_select(summ_np, q_np, gqa, n_blocks, n_recent, k_top):
    n_kv = summ_np.shape[0]
    geom = kv.Geom(n_kv, gqa, 1)
    out = kv.kvattn_select_blocks(geom, gpu(q_np), gpu(summ_np), summ_np.shape[1], n_blocks,
                                  n_recent, k_top)
    torch.cuda.synchronize()
    got = host(out)
    qs = oracle.query_sum(q_np, gqa)
    for h in range(n_kv):
        sc = oracle.block_scores(qs[h], summ_np[h, :n_blocks])
        ref = oracle.select_blocks(sc, n_blocks, n_recent, k_top)
        assert got.shape[1] == len(ref)
        assert (got[h] == ref).all(), f"head {h}: {got[h][:10]} vs {ref[:10]}"


@pytest.mark.parametrize("n_blocks,n_recent,k_top", [
    (300, 16, 40), (300, 16, 1), (300, 0, 299), (300, 299, 5), (300, 300, 5),
    (300, 400, 0), (300, 16, 0), (300, 16, 284), (300, 16, 1000), (4088, 128, 256),
    (2049, 3, 1024), (7, 2, 3)])
def test_select_bitexact(n_blocks, n_recent, k_top):
    g = np.random.default_rng(n_blocks + 7 * k_top)
    n_kv, gqa = 3, 6
    summ = (g.standard_normal((n_kv, n_blocks + 2, 256)) * 0.05).astype(np.float32)
    q = g.standard_normal((n_kv * gqa, 256)).astype(np.float32)
    run_select(summ, q, gqa, n_blocks, n_recent, k_top)


@pytest.mark.parametrize("n_kv,gqa,n_blocks,n_recent,k_top", [
    (3, 6, 300, 16, 40), (4, 6, 4088, 128, 256), (2, 1, 130, 0, 7), (1, 16, 700, 10, 100),
    (2, 9, 257, 3, 50), (1, 6, 65, 0, 1)])
def test_select_scores_bitexact(n_kv, gqa, n_blocks, n_recent, k_top):
    """The binary64 scores the ranking uses (left in the workspace from byte
    2048) equal the fixed-order sums bit for bit, including groups of more
    than eight query heads and a ragged last workgroup of candidates."""
    g = np.random.default_rng(n_blocks + gqa)
    summ = (g.standard_normal((n_kv, n_blocks, 256)) * 0.05).astype(np.float32)
    summ *= np.exp2(g.integers(-20, 20, (n_kv, n_blocks, 1))).astype(np.float32)
    q = g.standard_normal((n_kv * gqa, 256)).astype(np.float32)
    n_cand = n_blocks - min(n_recent, n_blocks)
    ws = torch.zeros(2048 + 8 * n_kv * n_cand + 4096, dtype=torch.uint8, device=DEV)
    kv.kvattn_select_blocks(kv.Geom(n_kv, gqa, 1), gpu(q), gpu(summ), n_blocks, n_blocks,
                            n_recent, k_top, workspace=ws)
    torch.cuda.synchronize()
    got = host(ws[2048:2048 + 8 * n_kv * n_cand]).view(np.float64).reshape(n_kv, n_cand)
    qs = oracle.query_sum(q, gqa)
    for h in range(n_kv):
        ref = np.asarray(oracle.block_scores(qs[h], summ[h, :n_cand]), np.float64)
        bad = np.flatnonzero(got[h].view(np.uint64) != ref.view(np.uint64))
        assert bad.size == 0, f"head {h}: {bad.size} scores differ, first {bad[:4]}"


def test_select_wide_range_and_many_candidates():
    """Scores of both signs spanning many binade (the radix select starts at
    the highest bit where candidates differ), and more candidates than the
    ranking keeps in LDS (keys re-read from the scores)."""
    g = np.random.default_rng(13)
    n_kv, gqa = 2, 6
    for nb, k in ((600, 50), (9000, 300), (12000, 7000)):
        summ = (g.standard_normal((n_kv, nb, 256)) * 0.05).astype(np.float32)
        summ *= np.exp2(g.integers(-40, 40, (n_kv, nb, 1))).astype(np.float32)
        q = g.standard_normal((n_kv * gqa, 256)).astype(np.float32)
        run_select(summ, q, gqa, nb, 16, k)
    # all candidates of one sign and magnitude but the last bits: a deep select
    summ = np.tile((g.standard_normal((n_kv, 1, 256)) * 0.05).astype(np.float32), (1, 700, 1))
    summ[:, :, 0] += np.float32(1e-6) * g.integers(0, 4, (n_kv, 700)).astype(np.float32)
    q = g.standard_normal((n_kv * gqa, 256)).astype(np.float32)
    run_select(summ, q, gqa, 700, 10, 123)


def test_select_ties_and_signed_zero():
    """Equal scores (duplicated summaries, zero summaries that score +0 and -0)
    go to the lowest block index."""
    g = np.random.default_rng(11)
    n_kv, gqa, nb = 2, 6, 500
    summ = (g.standard_normal((n_kv, nb, 256)) * 0.05).astype(np.float32)
    summ[:, 100:400:3] = summ[:, 50:51]                   # many exact ties
    summ[0, 7] = 0.0
    q = g.standard_normal((n_kv * gqa, 256)).astype(np.float32)
    for k in (1, 30, 60, 101, 200):
        run_select(summ, q, gqa, nb, 20, k)
    run_select(np.zeros_like(summ), q, gqa, nb, 20, 33)   # all scores 0 -> blocks 0..32


DECODE_CASES = [
    # n_q_tok, gqa, n_kv, kv_len, n_splits
    (1, 6, 2, 4096 + 77, 0),
    (4, 6, 2, 3000, 0),
    (2, 6, 1, 1500, 3),
    (1, 6, 1, 4096, 0),
    (1, 16, 1, 2000, 0),
    (1, 32, 1, 700, 5),
    (3, 5, 2, 777, 0),
    (4, 8, 1, 4, 0),
    (1, 1, 3, 130, 64),
    (1, 6, 1, 1100, 2),       # 9 pages over 2 splits: 4 and 5 (odd) per split
    (2, 16, 1, 2500, 0),      # 32 rows
    # one split over 193 pages: waves 4-7 take 72 units, waves 0-3 121, so
    # both halves reload their 64-unit page window; partial last page
    (4, 6, 2, 64 * 128 * 3 + 5, 1),
    (1, 6, 1, 300 * 128 - 40, 1),   # 300 pages, one split: windows reloaded twice
]


@pytest.mark.parametrize("n_q_tok,gqa,n_kv,kv_len,n_splits", DECODE_CASES)
def test_decode_dense(n_q_tok, gqa, n_kv, kv_len, n_splits):
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=kv_len + gqa, init_seed=5)
    q = np.random.default_rng(kv_len).standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16, n_splits=n_splits)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, len(table), kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o.reshape(n_q_tok, -1, 256), ref_l)
    assert eo <= DEC_TOL, eo
    assert el <= 1e-3 and rr <= 2e-3, (el, rr)


def test_decode_sparse_blocks():
    """Block lists (the selection output): a subset of pages including the
    partial last page, repeated calls with different lists, invalid entries."""
    n_kv, gqa, kv_len = 2, 6, 5000
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=21, init_seed=6)
    n_pages = len(table)
    g = np.random.default_rng(22)
    q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    lists = [
        np.stack([np.sort(g.choice(n_pages, 12, replace=False)) for _ in range(n_kv)]),
        np.stack([np.r_[np.sort(g.choice(n_pages - 1, 7, replace=False)), n_pages - 1]
                  for _ in range(n_kv)]),
        np.array([[0, -1, 5, 999, 39], [39, 38, 3, 2, -7]]),
    ]
    for blocks in lists:
        blocks = blocks.astype(np.int32)
        out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv,
                                    gpu(table, torch.int32), kv_len, 1 / 16,
                                    blocks=gpu(blocks, torch.int32))
        ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                     blocks=blocks)
        eo, el, rr = compare(out, lse, ref_o, ref_l)
        assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def indicator_pools(kv_len, n_phys, seed, n_kv=1, gqa=3):
    n_pages = (kv_len + 127) // 128
    K = np.zeros((kv_len, n_kv, 256), np.float32)
    V = np.zeros((kv_len, n_kv, 256), np.float32)
    V[np.arange(kv_len), :, (np.arange(kv_len) // 128) % 256] = 1.0
    table = np.random.default_rng(seed).permutation(n_phys)[:n_pages].astype(np.int32)
    pools = Pools(n_phys, n_kv, gqa, init_seed=seed)
    pools.write(K, V, 0, table)
    return pools, table


@pytest.mark.parametrize("n_q_tok", [1, 4])
def test_decode_indicator_exact(n_q_tok):
    """K = 0, V one-hot on dim (page mod 256): every softmax weight is 1, so
    o[n] = (#visible keys on pages == n) / (#visible keys) exactly, per row
    (causal among the verify tokens), dense and over a block list."""
    kv_len, gqa = 2000, 3
    pools, table = indicator_pools(kv_len, 20, 9, gqa=gqa)
    q = np.random.default_rng(1).standard_normal((n_q_tok, gqa, 256)).astype(np.float32)
    for blocks in (None, np.array([[15, 2, 7, 9]], np.int32)):
        out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv,
                                    gpu(table, torch.int32), kv_len, 1 / 16,
                                    blocks=None if blocks is None else gpu(blocks, torch.int32))
        o = host(out)
        pages = range(len(table)) if blocks is None else blocks[0]
        for t in range(n_q_tok):
            limit = kv_len - n_q_tok + t
            counts = np.zeros(256)
            for p in pages:
                counts[p % 256] += max(0, min(limit + 1, (p + 1) * 128) - p * 128)
            for gg in range(gqa):
                np.testing.assert_allclose(o[t, gg], counts / counts.sum(), rtol=0, atol=2e-7)
                assert abs(host(lse)[t, gg] - np.log(counts.sum())) < 1e-5


def test_decode_peaked_key_through_page_table():
    kv_len, n_phys, gqa = 3000, 40, 6
    g = np.random.default_rng(12)
    K = (g.standard_normal((kv_len, 1, 256)) * 0.01).astype(np.float32)
    V = g.standard_normal((kv_len, 1, 256)).astype(np.float32)
    q = g.standard_normal((1, gqa, 256)).astype(np.float32)
    j = 2222
    qsum = q[0].sum(axis=0)
    K[j, 0] = 40 * 16 * qsum / np.linalg.norm(qsum) / np.sqrt(gqa)
    table = g.permutation(n_phys)[:24].astype(np.int32)
    pools = Pools(n_phys, 1, gqa)
    pools.write(K, V, 0, table)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, 24, kv_len, 1 / 16)
    eo, el, _ = compare(out, lse, ref_o, ref_l)
    # s ~ 100 here: f16 operands (2^-11 relative) bound the lse error relatively
    assert eo <= DEC_TOL and el <= 2e-4 * np.abs(ref_l).max(), (eo, el)


def test_decode_deterministic_and_page_permutation_invariant():
    n_kv, gqa, kv_len = 2, 6, 3333
    pools, table, K, V = fill(n_kv, gqa, kv_len, seed=31)
    q = np.random.default_rng(32).standard_normal((4, n_kv * gqa, 256)).astype(np.float32)
    args = (pools.geom, gpu(q), pools.gk, pools.gv, gpu(table, torch.int32), kv_len, 1 / 16)
    o1, l1 = kv.kvattn_decode(*args)
    o2, l2 = kv.kvattn_decode(*args)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    table2 = np.random.default_rng(33).permutation(pools.n_phys)[:len(table)].astype(np.int32)
    pools2 = Pools(pools.n_phys, n_kv, gqa)
    pools2.write(K, V, 0, table2)
    o3, l3 = kv.kvattn_decode(pools2.geom, gpu(q), pools2.gk, pools2.gv,
                              gpu(table2, torch.int32), kv_len, 1 / 16)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_ten_launches_bit_identical():
    """Every kernel of the path sums in a fixed order, whatever the timing of
    the workgroups: ten launches of each give the same bits (verify shape,
    library-chosen splits; the append rewrites the same tokens each time;
    prefill with its page groups and counter waits)."""
    n_kv, gqa, kv_len = 4, 6, 64 * 128 + 37
    pools, table, K, V = fill(n_kv, gqa, kv_len, seed=51)
    g = np.random.default_rng(52)
    q = gpu(g.standard_normal((4, n_kv * gqa, 256)).astype(np.float32))
    t = gpu(table, torch.int32)
    first = None
    for i in range(10):
        o, l = kv.kvattn_decode(pools.geom, q, pools.gk, pools.gv, t, kv_len, 1 / 16)
        if first is None:
            first = (o.clone(), l.clone())
        assert torch.equal(o, first[0]) and torch.equal(l, first[1]), f"decode launch {i}"
    kn, vn = gpu(K[-4:]), gpu(V[-4:])
    first = None
    for i in range(10):
        o, l = kv.kvattn_append_decode(pools.geom, kn, vn, q, pools.gk, pools.gv, t, kv_len,
                                       1 / 16)
        if first is None:
            first = (o.clone(), l.clone())
        assert torch.equal(o, first[0]) and torch.equal(l, first[1]), f"append-decode launch {i}"
    chunk = 300
    qp = gpu(g.standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32))
    first = None
    for i in range(10):
        o, l = kv.kvattn_prefill_chunk(pools.geom, qp, pools.gk, pools.gv, t, kv_len - chunk,
                                       1 / 16)
        if first is None:
            first = (o.clone(), l.clone())
        assert torch.equal(o, first[0]) and torch.equal(l, first[1]), f"prefill launch {i}"


def test_merge_parity():
    """Partials with lse = -inf contribute nothing, whatever their rows hold
    (NaN here for the GPU; zeros for the oracle). Part counts cover every
    merge path: up to 64 parts (decode splits), one and several passes of the
    16-wave path, more parts than threads, and many rows with few parts."""
    g = np.random.default_rng(40)
    for S, rows, D in ((1, 5, 256), (7, 33, 256), (64, 96, 256), (63, 24, 256), (65, 6, 256),
                       (130, 7, 256), (300, 4, 100), (1100, 3, 256),
                       (16, 1501, 256), (3, 1024, 256), (32, 1100, 256)):  # last three: many rows
        o = g.standard_normal((S, rows, D)).astype(np.float32)
        ls = (g.standard_normal((S, rows)) * 3).astype(np.float32)
        ls[g.random((S, rows)) < 0.2] = -np.inf
        ls[:, 0] = -np.inf                                  # an all-empty row
        o[np.isneginf(ls)] = 0.0
        o_dev = o.copy()
        if D == 256:
            o_dev[np.isneginf(ls)] = np.nan
        out, lse = kv.kvattn_merge_lse(gpu(o_dev), gpu(ls))
        ref_o, ref_l = oracle.merge_lse(o, ls)
        got_o, got_l = host(out), host(lse)
        assert (got_o[0] == 0).all() and np.isneginf(got_l[0])
        np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=2e-5)
        fin = np.isfinite(ref_l)
        np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=2e-5)


PREFILL_CASES = [
    # chunk, pos0, gqa, n_kv, n_groups
    (70, 300, 6, 1, 0),
    (130, 1000, 6, 2, 3),
    (512, 2000, 6, 1, 0),
    (45, 0, 6, 1, 0),
    (200, 77, 4, 2, 1),
    (1, 555, 6, 1, 0),
]


@pytest.mark.parametrize("chunk,pos0,gqa,n_kv,n_groups", PREFILL_CASES)
def test_prefill_parity(chunk, pos0, gqa, n_kv, n_groups):
    kv_len = pos0 + chunk
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=chunk + pos0, init_seed=8)
    q = np.random.default_rng(kv_len).standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
    out, lse = prefill_checked(pools.geom, gpu(q), pools.gk, pools.gv,
                                       gpu(table, torch.int32), pos0, 1 / 16, n_groups=n_groups)
    ref_o, ref_l = oracle.prefill_chunk(q, gqa, pools.ok, pools.ov, table, len(table), pos0,
                                        1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= PRE_TOL, eo
    assert el <= 5e-3 and rr <= 5e-3, (el, rr)


def test_prefill_indicator_causal_exact():
    kv_len, pos0, gqa = 1500, 1100, 3
    pools, table = indicator_pools(kv_len, 14, 13, gqa=gqa)
    q = np.random.default_rng(2).standard_normal((kv_len - pos0, gqa, 256)).astype(np.float32)
    out, _ = prefill_checked(pools.geom, gpu(q), pools.gk, pools.gv,
                                     gpu(table, torch.int32), pos0, 1 / 16)
    o = host(out)
    for t in (0, 1, 27, 127, 128, 399):
        n = pos0 + t + 1
        counts = np.bincount(np.arange(n) // 128, minlength=256)[:256].astype(float)
        for gg in range(gqa):
            np.testing.assert_allclose(o[t, gg], counts / n, rtol=0, atol=2e-7)


@pytest.mark.gpu
def test_decode_partials_merge_to_decode():
    """kvattn_decode_partials + kvattn_merge_lse is kvattn_decode, bit for bit;
    each split's partial is attention over its own pages."""
    n_kv, gqa, kv_len, S = 2, 6, 5000, 7
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=31, init_seed=9)
    n_pages = len(table)
    for n_q_tok in (1, 4):
        q = np.random.default_rng(32 + n_q_tok).standard_normal(
            (n_q_tok, n_kv * gqa, 256)).astype(np.float32)
        qd, td = gpu(q), gpu(table, torch.int32)
        out, lse = kv.kvattn_decode(pools.geom, qd, pools.gk, pools.gv, td, kv_len, 1 / 16,
                                    n_splits=S)
        op, lp = kv.kvattn_decode_partials(pools.geom, qd, pools.gk, pools.gv, td, kv_len, 1 / 16,
                                           S)
        o2, l2 = kv.kvattn_merge_lse(op, lp)
        torch.cuda.synchronize()
        assert torch.equal(out.reshape(-1, 256), o2.reshape(-1, 256))
        assert torch.equal(lse.reshape(-1), l2.reshape(-1))
    # n_q_tok = 1: split s against the oracle over pages [n*s/S, n*(s+1)/S)
    q1 = np.random.default_rng(33).standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    op, lp = kv.kvattn_decode_partials(pools.geom, gpu(q1), pools.gk, pools.gv,
                                       gpu(table, torch.int32), kv_len, 1 / 16, S)
    opn, lpn = host(op), host(lp)
    for s in range(S):
        pages = np.arange(n_pages * s // S, n_pages * (s + 1) // S)
        blocks = np.stack([pages] * n_kv)
        ref_o, ref_l = oracle.decode(q1, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                     blocks=blocks)
        assert np.abs(opn[s] - ref_o.reshape(-1, 256)).max() <= DEC_TOL
        assert np.abs(lpn[s] - ref_l.reshape(-1)).max() <= 1e-3


@pytest.mark.gpu
def test_decode_partials_more_splits_than_pages():
    """Splits past the unit count are empty: o = 0, lse = -inf, and the merge
    still gives the oracle's result."""
    n_kv, gqa, kv_len, S = 1, 6, 700, 9          # 6 pages, 9 splits
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=34, init_seed=10)
    q = np.random.default_rng(35).standard_normal((1, gqa, 256)).astype(np.float32)
    op, lp = kv.kvattn_decode_partials(pools.geom, gpu(q), pools.gk, pools.gv,
                                       gpu(table, torch.int32), kv_len, 1 / 16, S)
    lpn = host(lp)
    empty = [s for s in range(S) if 6 * s // S == 6 * (s + 1) // S]
    assert empty and all(np.isneginf(lpn[s]).all() for s in empty)
    assert all((host(op)[s] == 0).all() for s in empty)
    o2, l2 = kv.kvattn_merge_lse(op, lp)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, len(table), kv_len, 1 / 16)
    eo, el, _ = compare(o2.reshape(1, gqa, 256), l2.reshape(1, gqa), ref_o.reshape(1, gqa, 256),
                        ref_l.reshape(1, gqa))
    assert eo <= DEC_TOL and el <= 1e-3


@pytest.mark.gpu
def test_prefill_partials_merge_to_prefill():
    chunk, pos0, gqa, n_kv, G = 130, 1000, 6, 2, 3
    kv_len = pos0 + chunk
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=36, init_seed=11)
    q = np.random.default_rng(37).standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
    qd, td = gpu(q), gpu(table, torch.int32)
    out, lse = prefill_checked(pools.geom, qd, pools.gk, pools.gv, td, pos0, 1 / 16,
                                       n_groups=G)
    op, lp = kv.kvattn_prefill_partials(pools.geom, qd, pools.gk, pools.gv, td, pos0, 1 / 16, G)
    o2, l2 = kv.kvattn_merge_lse(op, lp)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(-1, 256), o2.reshape(-1, 256))
    assert torch.equal(lse.reshape(-1), l2.reshape(-1))


@pytest.mark.gpu
def test_prefetch_pages_from_pinned_host():
    """a7: records of the listed physical pages arrive bit for bit in the
    device pool; other pages are untouched."""
    n_kv, n_phys = 2, 12
    g = kv.Geom(n_kv, 6, n_phys)
    rng = np.random.default_rng(40)
    hk = torch.from_numpy(rng.integers(0, 256, n_phys * n_kv * quant.K_RECORD_BYTES,
                                       dtype=np.uint8)).pin_memory()
    hv = torch.from_numpy(rng.integers(0, 256, n_phys * n_kv * quant.V_RECORD_BYTES,
                                       dtype=np.uint8)).pin_memory()
    dk = torch.zeros(hk.numel(), dtype=torch.uint8, device=DEV)
    dv = torch.zeros(hv.numel(), dtype=torch.uint8, device=DEV)
    pages = [3, 4, 5, 9, 0, 11]
    copy = torch.cuda.Stream()
    kv.kvattn_prefetch_pages(g, hk, hv, dk, dv, pages, stream=copy)
    copy.synchronize()
    K = host(dk).reshape(n_phys, -1)
    V = host(dv).reshape(n_phys, -1)
    HK, HV = hk.numpy().reshape(n_phys, -1), hv.numpy().reshape(n_phys, -1)
    for p_ in range(n_phys):
        if p_ in pages:
            assert (K[p_] == HK[p_]).all() and (V[p_] == HV[p_]).all(), p_
        else:
            assert not K[p_].any() and not V[p_].any(), p_


@pytest.mark.gpu
def test_decode_over_prefetched_staging_pool():
    """Layer-ahead streaming: the pool lives in pinned host memory, a copy
    stream fills a device staging pool, an event gates the decode; the result
    is the one decode gives on the device-resident pool, bit for bit."""
    n_kv, gqa, kv_len = 2, 6, 3000
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=41, init_seed=12)
    hk = torch.empty(pools.gk.numel(), dtype=torch.uint8, pin_memory=True)
    hv = torch.empty(pools.gv.numel(), dtype=torch.uint8, pin_memory=True)
    hk.copy_(pools.gk)
    hv.copy_(pools.gv)
    torch.cuda.synchronize()
    sk = torch.zeros_like(pools.gk)
    sv = torch.zeros_like(pools.gv)
    q = np.random.default_rng(42).standard_normal((4, n_kv * gqa, 256)).astype(np.float32)
    qd, td = gpu(q), gpu(table, torch.int32)
    copy = torch.cuda.Stream()
    ready = torch.cuda.Event()
    kv.kvattn_prefetch_pages(pools.geom, hk, hv, sk, sv, sorted(set(table.tolist())),
                             stream=copy)
    ready.record(copy)
    torch.cuda.current_stream().wait_event(ready)
    o1, l1 = kv.kvattn_decode(pools.geom, qd, sk, sv, td, kv_len, 1 / 16, n_splits=8)
    o2, l2 = kv.kvattn_decode(pools.geom, qd, pools.gk, pools.gv, td, kv_len, 1 / 16, n_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.gpu
def test_decode_window_reloads_one_split():
    """One split over hundreds of units, so each wave half reloads its 64-unit
    page window several times (units past 64, 128, ...): dense over 300
    pages through kvattn_decode and kvattn_decode_partials, a sparse list of
    260 blocks, and kvattn_append_decode over that list with the new tokens
    on its last block (found by the append's search past two reloads)."""
    n_kv, gqa, kv_len = 1, 6, 300 * 128 - 40
    pools, table, _, _ = fill(n_kv, gqa, kv_len, seed=91, init_seed=11)
    n_pages = len(table)
    g = np.random.default_rng(92)
    q = g.standard_normal((4, gqa, 256)).astype(np.float32)
    td = gpu(table, torch.int32)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, td, kv_len, 1 / 16,
                                n_splits=1)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o.reshape(4, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
    op, lp = kv.kvattn_decode_partials(pools.geom, gpu(q), pools.gk, pools.gv, td, kv_len, 1 / 16, 1)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(out.shape), out) and torch.equal(lp.reshape(lse.shape), lse)
    blocks = np.r_[np.sort(g.choice(n_pages - 1, 259, replace=False)), n_pages - 1]
    blocks = blocks[None, :].astype(np.int32)
    out, lse = kv.kvattn_decode(pools.geom, gpu(q), pools.gk, pools.gv, td, kv_len, 1 / 16,
                                blocks=gpu(blocks, torch.int32), n_splits=1)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                 blocks=blocks)
    eo, el, rr = compare(out, lse, ref_o.reshape(4, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
    # append four tokens at the end of the cache, attend over the same list
    n_new = 4
    Kn = g.standard_normal((n_new, n_kv, 256)).astype(np.float32)
    Vn = g.standard_normal((n_new, n_kv, 256)).astype(np.float32)
    out, lse = kv.kvattn_append_decode(pools.geom, gpu(Kn), gpu(Vn), gpu(q), pools.gk, pools.gv,
                                       td, kv_len + n_new, 1 / 16,
                                       blocks=gpu(blocks, torch.int32), n_splits=1)
    quant.quantize_into_pool(Kn, Vn, kv_len, table, pools.ok, pools.ov)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all() and (gv == pools.ov).all()
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len + n_new,
                                 1 / 16, blocks=blocks)
    eo, el, rr = compare(out, lse, ref_o.reshape(4, -1, 256), ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
