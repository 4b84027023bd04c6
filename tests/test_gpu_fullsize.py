"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (library-chosen splits and page groups, permuted page tables,
one layer's pool of the real shape).

The GPU computes every output; the oracle recomputes a sample it can finish
in seconds from the same seeded host inputs, quantising the sampled KV heads
itself (nothing the GPU produced is fed to it):
  - page bytes of sampled pages, bit for bit;
  - decode / verify outputs of one KV head (all its query rows);
  - prefill outputs of one KV head at sampled chunk positions;
  - KVMem summaries and selected blocks of two KV heads, bit for bit, the
    sparse decode of one head, and needle recall;
  - the verify step's fused append + decode: whole pools and outputs against
    quantise + decode bit for bit, one head against the oracle;
  - verify with the q8_0/q8_0 and q4_0/q4_0 caches: sampled pages, one head.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from long_context_attention_paged_amd import synth
from kvtest_util import DEV, compare, gpu, host, prefill_checked

pytestmark = pytest.mark.gpu

DEC_TOL, PRE_TOL = 2e-3, 1e-2
CHUNK = 32768  # tokens per quantisation call when filling a pool (as the benchmark does)


class FullLayer:
    """Layer 0 of workload w on the GPU, plus the host inputs it came from."""

    def __init__(self, w, summaries=False, k_type=0, v_type=0):
        self.w = w
        self.q = synth.queries(w, 0)
        self.K, self.V = synth.kv_layer(w, 0, self.q, threads=16)
        self.table = synth.page_table(w)
        self.geom = kv.Geom(w.n_kv, w.gqa, w.n_pages, v_type=v_type, k_type=k_type)
        self.k_rec, self.v_rec = self.geom.k_record_bytes, self.geom.v_record_bytes
        self.kp = torch.zeros(w.n_pages * w.n_kv * self.k_rec, dtype=torch.uint8, device=DEV)
        self.vp = torch.zeros(w.n_pages * w.n_kv * self.v_rec, dtype=torch.uint8, device=DEV)
        self.td = gpu(self.table, torch.int32)
        self.summ = (torch.zeros((w.n_kv, w.n_pages, 256), dtype=torch.float32, device=DEV)
                     if summaries else None)
        for a in range(0, w.kv_len, CHUNK):
            b = min(w.kv_len, a + CHUNK)
            kv.kvattn_quantize_pages(self.geom, gpu(self.K[a:b]), gpu(self.V[a:b]), a, self.td,
                                     self.kp, self.vp, self.summ)
        torch.cuda.synchronize()

    def oracle_pool(self, h):
        """The oracle's own pool for KV head h (n_kv = 1)."""
        w = self.w
        ok = np.zeros((w.n_pages, 1, self.k_rec), np.uint8)
        ov = np.zeros((w.n_pages, 1, self.v_rec), np.uint8)
        quant.quantize_into_pool(self.K[:, h:h + 1], self.V[:, h:h + 1], 0, self.table, ok, ov)
        return ok, ov

    def check_pages(self, pages):
        """Sampled pages: every KV head's records, bit for bit."""
        w = self.w
        gk = host(self.kp).reshape(w.n_pages, w.n_kv, -1)
        gv = host(self.vp).reshape(w.n_pages, w.n_kv, -1)
        for lp in pages:
            one = np.full(w.n_pages, -1, np.int32)
            one[lp] = 0
            ok = np.zeros((1, w.n_kv, self.k_rec), np.uint8)
            ov = np.zeros((1, w.n_kv, self.v_rec), np.uint8)
            sl = slice(lp * 128, min(w.kv_len, (lp + 1) * 128))
            quant.quantize_into_pool(self.K[sl], self.V[sl], lp * 128, one, ok, ov)
            ph = self.table[lp]
            assert (gk[ph] == ok[0]).all(), f"K page {lp}"
            assert (gv[ph] == ov[0]).all(), f"V page {lp}"


def sample_pages(w, rng):
    return sorted({0, w.n_pages - 1, *rng.choice(w.n_pages, 3, replace=False).tolist()})


def test_tiny_decode_4k_full():
    w = synth.WORKLOADS[1]
    L = FullLayer(w)
    L.check_pages(range(w.n_pages))
    out, lse = kv.kvattn_decode(L.geom, gpu(L.q), L.kp, L.vp, L.td, w.kv_len, 1 / 16)
    ok, ov = L.oracle_pool(0)
    ref_o, ref_l = oracle.decode(L.q, w.gqa, ok, ov, L.table, w.n_pages, w.kv_len, 1 / 16)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


@pytest.mark.parametrize("cfg,head", [(2, 1), (3, 2)])
def test_decode_full_size_one_head(cfg, head):
    """decode-131k (outlier channels) and verify-262k (4 causal query tokens)."""
    w = synth.WORKLOADS[cfg]
    L = FullLayer(w)
    L.check_pages(sample_pages(w, np.random.default_rng(cfg)))
    out, lse = kv.kvattn_decode(L.geom, gpu(L.q), L.kp, L.vp, L.td, w.kv_len, 1 / 16)
    torch.cuda.synchronize()
    ok, ov = L.oracle_pool(head)
    rows = slice(head * w.gqa, (head + 1) * w.gqa)
    ref_o, ref_l = oracle.decode(L.q[:, rows], w.gqa, ok, ov, L.table, w.n_pages, w.kv_len,
                                 1 / 16)
    eo, el, rr = compare(out[:, rows], lse[:, rows], ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


@pytest.mark.parametrize("k_type,v_type", [(kv.K_Q8_0, kv.V_Q8_0), (kv.K_Q4_0, kv.V_Q4_0),
                                            (kv.K_Q5_1, kv.V_Q4_0)])
def test_verify_full_size_other_pairs(k_type, v_type):
    """verify-262k with the q8_0/q8_0, q4_0/q4_0 and q5_1/q4_0 caches: sampled pages bit
    for bit, one KV head's outputs against the oracle."""
    w = synth.WORKLOADS[3]
    L = FullLayer(w, k_type=k_type, v_type=v_type)
    L.check_pages(sample_pages(w, np.random.default_rng(7 + k_type)))
    out, lse = kv.kvattn_decode(L.geom, gpu(L.q), L.kp, L.vp, L.td, w.kv_len, 1 / 16)
    torch.cuda.synchronize()
    head = (1 + k_type) % w.n_kv
    ok, ov = L.oracle_pool(head)
    rows = slice(head * w.gqa, (head + 1) * w.gqa)
    ref_o, ref_l = oracle.decode(L.q[:, rows], w.gqa, ok, ov, L.table, w.n_pages, w.kv_len,
                                 1 / 16)
    eo, el, rr = compare(out[:, rows], lse[:, rows], ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def test_prefill_full_size_sampled_tokens():
    """prefill-512-after-262k: KV head 3, chunk positions at both ends, at the
    page boundary inside the chunk and in the middle."""
    w = synth.WORKLOADS[4]
    head = 3
    L = FullLayer(w)
    L.check_pages(sample_pages(w, np.random.default_rng(4)) + [w.n_pages - 2])
    out, lse = prefill_checked(L.geom, gpu(L.q), L.kp, L.vp, L.td, w.pos0, 1 / 16)
    torch.cuda.synchronize()
    toks = [0, 1, 127, 128, 300, 510, 511]
    ok, ov = L.oracle_pool(head)
    rows = slice(head * w.gqa, (head + 1) * w.gqa)
    ref_o, ref_l = oracle.prefill_chunk(L.q[:, rows], w.gqa, ok, ov, L.table, w.n_pages, w.pos0,
                                        1 / 16, tokens=toks)
    eo, el, rr = compare(out[toks][:, rows], lse[toks][:, rows], ref_o[toks], ref_l[toks])
    assert eo <= PRE_TOL and el <= 5e-3 and rr <= 5e-3, (eo, el, rr)


def test_kvmem_full_size_selection_and_sparse_decode():
    w = synth.WORKLOADS[5]
    L = FullLayer(w, summaries=True)
    L.check_pages(sample_pages(w, np.random.default_rng(5)))
    n_out = kv.kvattn_select_count(w.n_pages, w.n_recent, w.k_top)
    blocks = torch.empty((w.n_kv, n_out), dtype=torch.int32, device=DEV)
    qd = gpu(L.q)
    kv.kvattn_select_blocks(L.geom, qd[-1], L.summ, w.n_pages, w.n_pages, w.n_recent, w.k_top,
                            out_blocks=blocks)
    out, lse = kv.kvattn_decode(L.geom, qd, L.kp, L.vp, L.td, w.kv_len, 1 / 16, blocks=blocks)
    torch.cuda.synchronize()
    gb = host(blocks)
    gs = host(L.summ)
    needles = synth.needle_blocks(w)
    for h in range(w.n_kv):  # recall: every needle block is selected for every head
        assert np.isin(needles, gb[h]).all(), h
    for h in (0, 3):
        ok, ov = L.oracle_pool(h)
        summ = quant.summaries_from_pool(ok, L.table, w.n_pages, 1)[0]
        assert (gs[h] == summ).all(), f"summaries of head {h}"
        rows = slice(h * w.gqa, (h + 1) * w.gqa)
        q_sel = oracle.query_sum(L.q[-1, rows], w.gqa)[0]
        sel = np.asarray(oracle.select_blocks(oracle.block_scores(q_sel, summ), w.n_pages,
                                              w.n_recent, w.k_top), np.int32)
        assert (gb[h] == sel).all(), f"selection of head {h}"
        if h == 0:
            ref_o, ref_l = oracle.decode(L.q[:, rows], w.gqa, ok, ov, L.table, w.n_pages,
                                         w.kv_len, 1 / 16, blocks=sel[None, :])
            eo, el, rr = compare(out[:, rows], lse[:, rows], ref_o, ref_l)
            assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)


def test_verify_full_size_append_decode():
    """verify-262k as the benchmark step runs it: one launch appends the 4 new
    tokens (fresh values, so the append changes the pool) and attends. Whole
    pools and outputs equal kvattn_quantize_pages + kvattn_decode bit for bit;
    KV head 1 matches the oracle over its own pool with the new tokens."""
    w = synth.WORKLOADS[3]
    head = 1
    L = FullLayer(w)
    g = np.random.default_rng(33)
    n_new = w.n_q_tok
    pos0 = w.kv_len - n_new
    Kn = g.standard_normal((n_new, w.n_kv, 256)).astype(np.float32)
    Vn = g.standard_normal((n_new, w.n_kv, 256)).astype(np.float32)
    kp2, vp2 = L.kp.clone(), L.vp.clone()
    kv.kvattn_quantize_pages(L.geom, gpu(Kn), gpu(Vn), pos0, L.td, kp2, vp2)
    o2, l2 = kv.kvattn_decode(L.geom, gpu(L.q), kp2, vp2, L.td, w.kv_len, 1 / 16)
    out, lse = kv.kvattn_append_decode(L.geom, gpu(Kn), gpu(Vn), gpu(L.q), L.kp, L.vp, L.td,
                                       w.kv_len, 1 / 16)
    torch.cuda.synchronize()
    assert torch.equal(L.kp, kp2) and torch.equal(L.vp, vp2), "pools differ"
    assert torch.equal(out, o2) and torch.equal(lse, l2), "outputs differ"
    K, V = L.K.copy(), L.V.copy()
    K[pos0:], V[pos0:] = Kn, Vn
    ok = np.zeros((w.n_pages, 1, quant.K_RECORD_BYTES), np.uint8)
    ov = np.zeros((w.n_pages, 1, quant.V_RECORD_BYTES), np.uint8)
    quant.quantize_into_pool(K[:, head:head + 1], V[:, head:head + 1], 0, L.table, ok, ov)
    rows = slice(head * w.gqa, (head + 1) * w.gqa)
    ref_o, ref_l = oracle.decode(L.q[:, rows], w.gqa, ok, ov, L.table, w.n_pages, w.kv_len, 1 / 16)
    eo, el, rr = compare(out[:, rows], lse[:, rows], ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
