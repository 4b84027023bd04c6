"""GPU parity of adaptive host-resident KV streaming (streaming.StreamedDecode):
the newest pages stay on the device and take the appended tokens, the older
history streams from pinned host memory every step, and the LSE merge of the
two equals attention over the whole cache (oracle, decode bar 2e-3). The
resident pool's bytes after the append equal the oracle's quantisation bit for
bit; repeated steps give identical results."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from long_context_attention_paged_amd import streaming
from kvtest_util import DEV, Pools, compare, gpu, host

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3


@pytest.mark.parametrize("k_type,v_type", [(0, 0), (1, 1)])  # q8_0/q4_0 and q4_0/q8_0 caches
@pytest.mark.parametrize("n_kv,gqa,n_q_tok,kv_len,n_hist,n_layers", [
    (2, 6, 4, 40 * 128 - 50, 28, 3),   # verify: history + resident, three layers (both slots)
    (1, 6, 1, 9 * 128 + 1, 8, 2),      # decode: the new token opens the resident last page
    (2, 6, 4, 12 * 128, 0, 2),         # no history: everything resident
])
def test_streamed_decode_matches_oracle(n_kv, gqa, n_q_tok, kv_len, n_hist, n_layers, k_type,
                                        v_type):
    g = np.random.default_rng(kv_len + n_hist)
    n_pages = (kv_len + 127) // 128
    n_phys = n_pages + 2
    pos0 = kv_len - n_q_tok
    geom = kv.Geom(n_kv, gqa, n_phys, v_type=v_type, k_type=k_type)
    layers, pools, tables, qs, kns, vns = [], [], [], [], [], []
    for _ in range(n_layers):
        table = g.permutation(n_phys)[:n_pages].astype(np.int32)
        p = Pools(n_phys, n_kv, gqa, init_seed=int(g.integers(1 << 30)), v_type=v_type,
                  k_type=k_type)
        p.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
        layers.append(streaming.StreamedLayer(geom, p.gk, p.gv, gpu(table, torch.int32), n_pages,
                                              n_hist))
        pools.append(p)
        tables.append(table)
        qs.append(g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32))
        kns.append(g.standard_normal((n_q_tok, n_kv, 256)).astype(np.float32))
        vns.append(g.standard_normal((n_q_tok, n_kv, 256)).astype(np.float32))
    sd = streaming.StreamedDecode(geom, layers, n_pages, n_q_tok, DEV)
    q_d, k_d, v_d = [gpu(x) for x in qs], [gpu(x) for x in kns], [gpu(x) for x in vns]
    outs = [torch.empty_like(x) for x in q_d]
    lses = [torch.empty(x.shape[:2], dtype=torch.float32, device=DEV) for x in q_d]
    sd.step(q_d, k_d, v_d, kv_len, 1 / 16, outs, lses)
    torch.cuda.synchronize()
    first = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    sd.step(q_d, k_d, v_d, kv_len, 1 / 16, outs, lses)  # same tokens again: same bytes, same result
    torch.cuda.synchronize()
    for c in range(n_layers):
        assert torch.equal(outs[c], first[c][0]) and torch.equal(lses[c], first[c][1])
        p, table = pools[c], tables[c]
        quant.quantize_into_pool(kns[c], vns[c], pos0, table, p.ok, p.ov)
        L = layers[c]
        rk = host(L.res_k).reshape(L.n_res, n_kv, -1)
        rv = host(L.res_v).reshape(L.n_res, n_kv, -1)
        assert (rk == p.ok[table[n_hist:]]).all() and (rv == p.ov[table[n_hist:]]).all()
        ref_o, ref_l = oracle.decode(qs[c], gqa, p.ok, p.ov, table, n_pages, kv_len, 1 / 16)
        eo, el, rr = compare(outs[c], lses[c], ref_o, ref_l)
        assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (c, eo, el, rr)
    assert sd.host_to_device_bytes_per_step() == n_layers * n_hist * n_kv * (
        geom.k_record_bytes + geom.v_record_bytes)



@pytest.mark.parametrize("src_on_host", [True, False])
def test_gather_blocks_bitexact(src_on_host):
    """kvattn_gather_blocks copies each kept block's records to its rank slot
    bit for bit, from pinned host memory or from the device, marks entries
    outside the table or the pool -1 and leaves their slots untouched."""
    n_kv, n_phys, n_logical, n_blk, n_sel = 3, 20, 18, 10, 8
    g = np.random.default_rng(5 + src_on_host)
    pools = Pools(n_phys, n_kv, 6, init_seed=9)
    table = g.permutation(n_phys)[:n_logical].astype(np.int32)
    table[5] = 99                                      # maps outside the pool
    blocks = np.stack([g.permutation(n_logical)[:n_blk] for _ in range(n_kv)]).astype(np.int32)
    blocks[0, 1], blocks[1, 2], blocks[2, 0] = -1, 30, 5   # invalid entries
    if src_on_host:
        sk = torch.empty(pools.gk.numel(), dtype=torch.uint8, pin_memory=True)
        sv = torch.empty(pools.gv.numel(), dtype=torch.uint8, pin_memory=True)
        sk.copy_(pools.gk)
        sv.copy_(pools.gv)
    else:
        sk, sv = pools.gk, pools.gv
    dk = torch.full((n_sel * n_kv * quant.K_RECORD_BYTES,), 0xAB, dtype=torch.uint8, device=DEV)
    dv = torch.full((n_sel * n_kv * quant.V_RECORD_BYTES,), 0xAB, dtype=torch.uint8, device=DEV)
    db = kv.kvattn_gather_blocks(pools.geom, sk, sv, gpu(table, torch.int32),
                                 gpu(blocks, torch.int32), n_sel, dk, dv)
    torch.cuda.synchronize()
    got_k = host(dk).reshape(n_sel, n_kv, -1)
    got_v = host(dv).reshape(n_sel, n_kv, -1)
    got_b = host(db)
    for h in range(n_kv):
        for i in range(n_sel):
            lp = blocks[h, i]
            ok = 0 <= lp < n_logical and 0 <= table[lp] < n_phys
            assert got_b[h, i] == (i if ok else -1)
            if ok:
                assert (got_k[i, h] == pools.ok[table[lp], h]).all()
                assert (got_v[i, h] == pools.ov[table[lp], h]).all()
            else:
                assert (got_k[i, h] == 0xAB).all() and (got_v[i, h] == 0xAB).all()


def test_kvmem_host_tier_matches_oracle():
    """KVMem with the history in pinned host memory: per layer the kept blocks
    (selected on the device, bit-exact with the oracle's selection) are pulled
    over the host link and attended with the resident recent window; the
    result equals the oracle's attention over the selection."""
    n_kv, gqa, n_pages, n_recent, k_top = 2, 6, 40, 8, 10
    kv_len = n_pages * 128                           # the new token completes the last page
    n_phys = n_pages + 2
    g = np.random.default_rng(123)
    geom = kv.Geom(n_kv, gqa, n_phys)
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    pools = Pools(n_phys, n_kv, gqa, init_seed=7)
    summ = torch.zeros((n_kv, n_pages, 256), dtype=torch.float32, device=DEV)
    pools.write(g.standard_normal((kv_len - 1, n_kv, 256)).astype(np.float32),
                g.standard_normal((kv_len - 1, n_kv, 256)).astype(np.float32), 0, table, summ)
    table_d = gpu(table, torch.int32)
    layer = streaming.KVMemHostLayer(geom, pools.gk, pools.gv, table_d, n_pages, n_recent, summ)
    kd = streaming.KVMemHostDecode(geom, [layer], table_d, n_pages, n_recent, k_top, 1, DEV)
    q = g.standard_normal((1, n_kv * gqa, 256)).astype(np.float32)
    kn = g.standard_normal((1, n_kv, 256)).astype(np.float32)
    vn = g.standard_normal((1, n_kv, 256)).astype(np.float32)
    out = torch.empty((1, n_kv * gqa, 256), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, n_kv * gqa), dtype=torch.float32, device=DEV)
    kd.step([gpu(q)], [gpu(kn)], [gpu(vn)], kv_len, 1 / 16, [out], [lse])
    torch.cuda.synchronize()
    kept = host(kd.kept[0])
    # the selection ran on the summaries before this step's append (the last
    # page is in the recent window, not a candidate)
    qs = oracle.query_sum(q[0], gqa)
    summ_ref = quant.summaries_from_pool(pools.ok, table, n_pages - 1, n_kv)
    for h in range(n_kv):
        sc = oracle.block_scores(qs[h], summ_ref[h, :n_pages - n_recent])
        ref = oracle.select_blocks(np.r_[sc, np.zeros(n_recent)], n_pages, n_recent, k_top)
        assert (kept[h] == ref).all(), (h, kept[h], ref)
    quant.quantize_into_pool(kn, vn, kv_len - 1, table, pools.ok, pools.ov)
    ref_o, ref_l = oracle.decode(q, gqa, pools.ok, pools.ov, table, n_pages, kv_len, 1 / 16,
                                 blocks=kept)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
    # the append completed the last page: its summary now matches the oracle's
    full = quant.summaries_from_pool(pools.ok, table, n_pages, n_kv)
    got = host(summ)
    assert (got[:, n_pages - 1].view(np.uint32) == full[:, n_pages - 1].view(np.uint32)).all()


@pytest.mark.parametrize("k_type,v_type", [(0, 0), (2, 1)])  # q8_0/q4_0 and q5_1/q8_0 caches
def test_host_pool_prefill_matches_oracle(k_type, v_type):
    """streaming.HostPoolPrefill (a7): three layers whose pools live only in
    pinned host memory, two consecutive chunks. Each chunk's out and lse match
    the oracle's prefill over the oracle's pool (prefill bar 1e-2 max-abs),
    and the host pools afterwards equal the oracle's quantisation bit for bit.
    The second chunk reads the first chunk's tokens from the host pools, where
    only the write-back put them; every workspace error word stays 0."""
    n_kv, gqa, n_layers = 2, 6, 3
    pos0, chunk0, chunk1 = 36 * 128 + 50, 200, 150
    n_pages = (pos0 + chunk0 + chunk1 + 127) // 128
    n_phys = n_pages + 2
    g = np.random.default_rng(70 + k_type)
    geom = kv.Geom(n_kv, gqa, n_phys, v_type=v_type, k_type=k_type)
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    pools, host_k, host_v = [], [], []
    for _ in range(n_layers):
        p = Pools(n_phys, n_kv, gqa, init_seed=int(g.integers(1 << 30)), v_type=v_type,
                  k_type=k_type)
        p.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
        torch.cuda.synchronize()
        hk = torch.empty(p.gk.numel(), dtype=torch.uint8, pin_memory=True)
        hv = torch.empty(p.gv.numel(), dtype=torch.uint8, pin_memory=True)
        hk.copy_(p.gk)
        hv.copy_(p.gv)
        p.gk = p.gv = None  # the device pools are gone: the host pools are the cache
        pools.append(p)
        host_k.append(hk)
        host_v.append(hv)
    hp = streaming.HostPoolPrefill(geom, host_k, host_v, table, DEV)
    start = pos0
    for chunk in (chunk0, chunk1):
        qs = [g.standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
              for _ in range(n_layers)]
        kns = [g.standard_normal((chunk, n_kv, 256)).astype(np.float32) for _ in range(n_layers)]
        vns = [g.standard_normal((chunk, n_kv, 256)).astype(np.float32) for _ in range(n_layers)]
        outs = [torch.empty((chunk, n_kv * gqa, 256), dtype=torch.float32, device=DEV)
                for _ in range(n_layers)]
        lses = [torch.empty((chunk, n_kv * gqa), dtype=torch.float32, device=DEV)
                for _ in range(n_layers)]
        print(f"host-pool prefill: chunk {chunk} at {start}", flush=True)
        hp.step([gpu(x) for x in qs], [gpu(x) for x in kns], [gpu(x) for x in vns], start,
                1 / 16, outs, lses)
        torch.cuda.synchronize()
        assert kv.workspace_error(hp.ws) == 0
        for c in range(n_layers):
            p = pools[c]
            quant.quantize_into_pool(kns[c], vns[c], start, table, p.ok, p.ov)
            assert (host(host_k[c]).reshape(p.ok.shape) == p.ok).all()
            assert (host(host_v[c]).reshape(p.ov.shape) == p.ov).all()
            ref_o, ref_l = oracle.prefill_chunk(qs[c], gqa, p.ok, p.ov, table, n_pages, start,
                                                1 / 16)
            eo, el, rr = compare(outs[c], lses[c], ref_o, ref_l)
            assert eo <= 1e-2 and el <= 1e-2, (chunk, c, eo, el, rr)
        start += chunk


@pytest.mark.parametrize("k_type,v_type", [(0, 0), (1, 1)])  # q8_0/q4_0 and q4_0/q8_0 caches
def test_budgeted_host_prefill_matches_oracle(k_type, v_type):
    """streaming.BudgetedHostPrefill: each layer's pages only in a pinned host
    tier (logical page order), a device budget of two 15-page staging slots,
    so each layer's pages go through three ranges (one copy per pool each,
    kvattn_prefill_range_partials per range, kvattn_merge_lse); two
    consecutive chunks over three layers. Out and lse match the oracle's
    prefill (1e-2 max-abs), the host tier afterwards equals the oracle's
    quantisation bit for bit, and the second chunk reads the first chunk's
    tokens from the host tier."""
    n_kv, gqa, n_layers = 2, 6, 3
    pos0, chunk0, chunk1 = 36 * 128 + 50, 200, 150
    n_pages = (pos0 + chunk0 + chunk1 + 127) // 128
    n_phys = n_pages + 2
    g = np.random.default_rng(80 + k_type)
    geom = kv.Geom(n_kv, gqa, n_phys, v_type=v_type, k_type=k_type)
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    pools, host_k, host_v = [], [], []
    for _ in range(n_layers):
        p = Pools(n_phys, n_kv, gqa, init_seed=int(g.integers(1 << 30)), v_type=v_type,
                  k_type=k_type)
        p.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
        torch.cuda.synchronize()
        # the host tier in logical page order: page p's records at p * n_kv
        tl = torch.from_numpy(table.astype(np.int64)).to(DEV)
        hk = torch.empty(n_pages * n_kv * geom.k_record_bytes, dtype=torch.uint8,
                         pin_memory=True)
        hv = torch.empty(n_pages * n_kv * geom.v_record_bytes, dtype=torch.uint8,
                         pin_memory=True)
        hk.copy_(p.gk.view(n_phys, -1)[tl].reshape(-1))
        hv.copy_(p.gv.view(n_phys, -1)[tl].reshape(-1))
        p.gk = p.gv = None
        pools.append(p)
        host_k.append(hk)
        host_v.append(hv)
    page_bytes = n_kv * (geom.k_record_bytes + geom.v_record_bytes)
    bp = streaming.BudgetedHostPrefill(geom, host_k, host_v, n_pages, DEV,
                                       budget_bytes=2 * 15 * page_bytes)
    assert bp.slot_pages == 15 and bp.device_bytes() == 2 * 15 * page_bytes
    start = pos0
    for chunk in (chunk0, chunk1):
        rng = bp.ranges(start, chunk)
        assert len(rng) == 3 and rng[0][0] == 0 and rng[-1][1] == (start + chunk + 127) // 128
        assert all(a < b <= a + 15 for a, b in rng)
        assert all(rng[i][1] == rng[i + 1][0] for i in range(len(rng) - 1))
        qs = [g.standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
              for _ in range(n_layers)]
        kns = [g.standard_normal((chunk, n_kv, 256)).astype(np.float32) for _ in range(n_layers)]
        vns = [g.standard_normal((chunk, n_kv, 256)).astype(np.float32) for _ in range(n_layers)]
        outs = [torch.empty((chunk, n_kv * gqa, 256), dtype=torch.float32, device=DEV)
                for _ in range(n_layers)]
        lses = [torch.empty((chunk, n_kv * gqa), dtype=torch.float32, device=DEV)
                for _ in range(n_layers)]
        print(f"budgeted prefill: chunk {chunk} at {start}, ranges {rng}", flush=True)
        bp.step([gpu(x) for x in qs], [gpu(x) for x in kns], [gpu(x) for x in vns], start,
                1 / 16, outs, lses)
        torch.cuda.synchronize()
        for c in range(n_layers):
            p = pools[c]
            quant.quantize_into_pool(kns[c], vns[c], start, table, p.ok, p.ov)
            # the host tier holds the oracle's pool in logical page order
            assert (host(host_k[c]).reshape(n_pages, n_kv, -1) == p.ok[table]).all()
            assert (host(host_v[c]).reshape(n_pages, n_kv, -1) == p.ov[table]).all()
            ref_o, ref_l = oracle.prefill_chunk(qs[c], gqa, p.ok, p.ov, table, n_pages, start,
                                                1 / 16)
            eo, el, rr = compare(outs[c], lses[c], ref_o, ref_l)
            assert eo <= 1e-2 and el <= 1e-2, (chunk, c, eo, el, rr)
        start += chunk


def test_prefill_range_partials_tile_the_chunk():
    """kvattn_prefill_range_partials over ranges that tile the chunk's pages
    (one of them holding a single page, one the causal tail), merged with
    kvattn_merge_lse, against the oracle and against kvattn_prefill_chunk;
    the last range, whose keys all lie past the causal limit of the chunk's
    early rows, gives those rows lse = -inf."""
    n_kv, gqa = 2, 6
    pos0, chunk = 9 * 128 + 17, 160
    n_pages = (pos0 + chunk + 127) // 128
    g = np.random.default_rng(33)
    table = g.permutation(n_pages + 1)[:n_pages].astype(np.int32)
    pools = Pools(n_pages + 1, n_kv, gqa, init_seed=34)
    pools.write(g.standard_normal((pos0 + chunk, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0 + chunk, n_kv, 256)).astype(np.float32), 0, table)
    q = g.standard_normal((chunk, n_kv * gqa, 256)).astype(np.float32)
    qd, td = gpu(q), gpu(table, torch.int32)
    parts, lparts = [], []
    for a, b, gr in [(0, 4, 3), (4, 5, 2), (5, 10, 2), (10, n_pages, 1)]:
        o, l_ = kv.kvattn_prefill_range_partials(pools.geom, qd, pools.gk, pools.gv, td, pos0,
                                                 1 / 16, a, b, gr)
        parts.append(o)
        lparts.append(l_)
    o_all, l_all = torch.cat(parts), torch.cat(lparts)
    out, lse = kv.kvattn_merge_lse(o_all, l_all)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.prefill_chunk(q, gqa, pools.ok, pools.ov, table, n_pages, pos0, 1 / 16)
    eo, el, rr = compare(out.view(chunk, -1, 256), lse.view(chunk, -1), ref_o, ref_l)
    assert eo <= 1e-2 and el <= 1e-2, (eo, el, rr)
    o2, l2 = kv.kvattn_prefill_chunk(pools.geom, qd, pools.gk, pools.gv, td, pos0, 1 / 16)
    assert (out.view_as(o2) - o2).abs().max().item() <= 2e-3
    # the last range [10, n_pages) holds only keys at positions >= 1280 > pos0:
    # query token t sees them only if pos0 + t >= 1280
    l_last = host(lparts[-1]).reshape(chunk, -1)
    first_seen = 10 * 128 - pos0
    assert np.isneginf(l_last[:first_seen]).all() and np.isfinite(l_last[first_seen:]).all()
