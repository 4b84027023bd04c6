"""Pins for the oracle's attention (decode, verify, prefill) and LSE merge.

Independent references: torch's float64 scaled_dot_product_attention and
logsumexp on the CPU, closed forms (zero query, constant values, single key,
indicator pages), the LSE-merge identity over arbitrary page splits, and a
peaked key that exposes the page-table indirection.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from long_context_attention_paged_amd import synth

D = 256


def make_pool(K, V, table, n_phys):
    n_tok, n_kv, _ = K.shape
    kp = np.zeros((n_phys, n_kv, quant.K_RECORD_BYTES), np.uint8)
    vp = np.zeros((n_phys, n_kv, quant.V_RECORD_BYTES), np.uint8)
    quant.quantize_into_pool(K, V, 0, table, kp, vp)
    return kp, vp


def direct_dequant(K, V):
    """Dequantised K, V [n_tok, n_kv, 256] straight from the block quantisers
    (no pages, no layout)."""
    n_tok, n_kv, _ = K.shape
    kc, kb = quant.q8_0_quantize(K.reshape(n_tok, n_kv, 8, 32))
    vc, vb = quant.q4_0_quantize(V.reshape(n_tok, n_kv, 8, 32))
    return (quant.q8_0_dequantize(kc, kb).reshape(n_tok, n_kv, D),
            quant.q4_0_dequantize(vc, vb).reshape(n_tok, n_kv, D))


def torch_ref(q_rows, khat, vhat, limits, pos, scale):
    """float64 SDPA and logsumexp on the CPU, boolean mask pos <= limit."""
    q = torch.tensor(q_rows, dtype=torch.float64)[None, None]
    k = torch.tensor(khat, dtype=torch.float64)[None, None]
    v = torch.tensor(vhat, dtype=torch.float64)[None, None]
    mask = torch.tensor(pos[None, :] <= np.asarray(limits)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None],
                                                         scale=scale)[0, 0]
    s = scale * (q[0, 0] @ k[0, 0].T)
    s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("n_q_tok,kv_len", [(1, 1000), (4, 777), (3, 512)])
def test_decode_matches_torch_sdpa(n_q_tok, kv_len):
    """Paged decode/verify through a permuted page table equals float64 SDPA on
    the directly dequantised, unpaged keys (causal among the query tokens)."""
    gqa, n_kv = 6, 2
    K, V, Q = synth.small_case(11 + n_q_tok, kv_len, n_kv, n_q_tok, gqa)
    n_pages = (kv_len + 127) // 128
    table = np.random.default_rng(3).permutation(n_pages + 2)[:n_pages].astype(np.int32)
    kp, vp = make_pool(K, V, table, n_pages + 2)
    out, lse = oracle.decode(Q, gqa, kp, vp, table, n_pages, kv_len, 1 / 16)
    kh, vh = direct_dequant(K, V)
    pos = np.arange(kv_len)
    for h in range(n_kv):
        rows = Q[:, h * gqa:(h + 1) * gqa].reshape(-1, D)
        lim = np.repeat(kv_len - n_q_tok + np.arange(n_q_tok), gqa)
        o_ref, l_ref = torch_ref(rows, kh[:, h], vh[:, h], lim, pos, 1 / 16)
        np.testing.assert_allclose(out[:, h * gqa:(h + 1) * gqa].reshape(-1, D), o_ref,
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, h * gqa:(h + 1) * gqa].reshape(-1), l_ref,
                                   rtol=0, atol=1e-12)


def test_prefill_matches_torch_sdpa():
    gqa, n_kv, pos0, chunk = 6, 1, 300, 70
    K, V, Q = synth.small_case(21, pos0 + chunk, n_kv, chunk, gqa)
    n_pages = (pos0 + chunk + 127) // 128
    table = np.arange(n_pages, dtype=np.int32)[::-1].copy()
    kp, vp = make_pool(K, V, table, n_pages)
    out, lse = oracle.prefill_chunk(Q, gqa, kp, vp, table, n_pages, pos0, 0.0625)
    kh, vh = direct_dequant(K, V)
    rows = Q.reshape(-1, D)
    lim = np.repeat(pos0 + np.arange(chunk), gqa)
    o_ref, l_ref = torch_ref(rows, kh[:, 0], vh[:, 0], lim, np.arange(pos0 + chunk), 0.0625)
    np.testing.assert_allclose(out.reshape(-1, D), o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(-1), l_ref, rtol=0, atol=1e-12)


def test_lse_merge_identity_any_split():
    """Attention over a random split of the pages, merged by LSE, equals
    attention over all pages ([RDNA4] online LSE accumulation)."""
    gqa, n_kv, kv_len = 6, 1, 1300
    K, V, Q = synth.small_case(31, kv_len, n_kv, 4, gqa)
    n_pages = 11
    table = np.arange(n_pages, dtype=np.int32)
    kp, vp = make_pool(K, V, table, n_pages)
    full_o, full_l = oracle.decode(Q, gqa, kp, vp, table, n_pages, kv_len, 1 / 16)
    g = np.random.default_rng(4)
    for n_parts in (2, 3, 5):
        assign = g.integers(0, n_parts, n_pages)
        parts_o, parts_l = [], []
        for s in range(n_parts):
            blocks = np.nonzero(assign == s)[0][None, :]
            o, l_ = oracle.decode(Q, gqa, kp, vp, table, n_pages, kv_len, 1 / 16, blocks=blocks)
            parts_o.append(o.reshape(-1, D))
            parts_l.append(l_.reshape(-1))
        mo, ml = oracle.merge_lse(np.stack(parts_o), np.stack(parts_l))
        np.testing.assert_allclose(mo, full_o.reshape(-1, D), rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, full_l.reshape(-1), rtol=0, atol=1e-12)


def test_closed_forms():
    gqa, n_kv, kv_len = 2, 1, 300
    K, V, Q = synth.small_case(41, kv_len, n_kv, 1, gqa)
    table = np.arange(3, dtype=np.int32)
    # zero query: o = mean of Vhat, lse = ln n
    kp, vp = make_pool(K, V, table, 3)
    o, l_ = oracle.decode(np.zeros_like(Q), gqa, kp, vp, table, 3, kv_len, 1 / 16)
    _, vh = direct_dequant(K, V)
    np.testing.assert_allclose(o[0, 0], vh[:, 0].mean(axis=0), rtol=0, atol=1e-13)
    assert abs(l_[0, 0] - np.log(kv_len)) < 1e-13
    # constant values (exact in Q4_0): softmax weights sum to one -> o = value
    Vc = np.full_like(V, 0.75)
    kp, vp = make_pool(K, Vc, table, 3)
    o, _ = oracle.decode(Q, gqa, kp, vp, table, 3, kv_len, 1 / 16)
    np.testing.assert_allclose(o, 0.75, rtol=0, atol=1e-14)
    # a single key: o = Vhat_0, lse = s_0
    kp, vp = make_pool(K[:1], V[:1], table, 3)
    o, l_ = oracle.decode(Q, gqa, kp, vp, table, 3, 1, 1 / 16)
    kh, vh = direct_dequant(K[:1], V[:1])
    np.testing.assert_allclose(o[0, 0], vh[0, 0], rtol=0, atol=0)
    assert abs(l_[0, 0] - Q[0, 0].astype(np.float64) @ kh[0, 0] / 16) < 1e-13


def indicator_case(kv_len, n_phys, seed):
    """K = 0; V_t[n] = 1 iff n == logical page of t (mod 256); exact in Q4_0.
    Then o[n] = (# visible keys on pages == n mod 256) / (# visible keys)."""
    n_pages = (kv_len + 127) // 128
    K = np.zeros((kv_len, 1, D), np.float32)
    V = np.zeros((kv_len, 1, D), np.float32)
    V[np.arange(kv_len), 0, (np.arange(kv_len) // 128) % 256] = 1.0
    table = np.random.default_rng(seed).permutation(n_phys)[:n_pages].astype(np.int32)
    kp, vp = make_pool(K, V, table, n_phys)
    return kp, vp, table, n_pages


@pytest.mark.parametrize("n_q_tok", [1, 4])
def test_indicator_pages_dense_and_sparse(n_q_tok):
    kv_len = 1000
    kp, vp, table, n_pages = indicator_case(kv_len, 12, 5)
    gqa = 3
    Q = np.random.default_rng(6).standard_normal((n_q_tok, gqa, D)).astype(np.float32)
    for blocks in (None, np.array([[7, 2, 5]]), np.array([[0, 7, 99, -1]])):
        o, l_ = oracle.decode(Q, gqa, kp, vp, table, n_pages, kv_len, 1 / 16, blocks=blocks)
        pages = range(n_pages) if blocks is None else [b for b in blocks[0] if 0 <= b < n_pages]
        for t in range(n_q_tok):
            limit = kv_len - n_q_tok + t
            counts = np.zeros(D)
            for p in pages:
                counts[p % 256] += max(0, min(limit + 1, (p + 1) * 128) - p * 128)
            for g in range(gqa):
                np.testing.assert_allclose(o[t, g], counts / counts.sum(), rtol=0, atol=1e-15)
                assert abs(l_[t, g] - np.log(counts.sum())) < 1e-12


def test_indicator_prefill_causal():
    kv_len, pos0 = 700, 600
    kp, vp, table, n_pages = indicator_case(kv_len, 6, 7)
    Q = np.random.default_rng(8).standard_normal((kv_len - pos0, 2, D)).astype(np.float32)
    o, _ = oracle.prefill_chunk(Q, 2, kp, vp, table, n_pages, pos0, 1 / 16)
    for t in (0, 1, 55, 99):
        n = pos0 + t + 1
        counts = np.bincount(np.arange(n) // 128, minlength=D)[:D].astype(float)
        np.testing.assert_allclose(o[t, 1], counts / n, rtol=0, atol=1e-15)


def test_peaked_key_follows_page_table():
    """One key 40*q/|q| on a page placed at a random physical slot; the output
    is that token's value (all other weights are < e^-300 relative)."""
    kv_len, n_phys = 900, 10
    g = np.random.default_rng(9)
    K = (g.standard_normal((kv_len, 1, D)) * 0.01).astype(np.float32)
    V = g.standard_normal((kv_len, 1, D)).astype(np.float32)
    Q = g.standard_normal((1, 1, D)).astype(np.float32)
    j = 517
    K[j, 0] = 40 * Q[0, 0] / np.linalg.norm(Q[0, 0]) * 16
    n_pages = 8
    table = g.permutation(n_phys)[:n_pages].astype(np.int32)
    kp, vp = make_pool(K, V, table, n_phys)
    o, _ = oracle.decode(Q, 1, kp, vp, table, n_pages, kv_len, 1 / 16)
    _, vh = direct_dequant(K, V)
    np.testing.assert_allclose(o[0, 0], vh[j, 0], rtol=0, atol=1e-12)


def test_merge_properties():
    g = np.random.default_rng(10)
    o = g.standard_normal((3, 5, 8))
    ls = g.standard_normal((3, 5))
    mo, ml = oracle.merge_lse(o[:1], ls[:1])
    np.testing.assert_array_equal(mo, o[0])
    np.testing.assert_array_equal(ml, ls[0])
    # a -inf part is neutral
    o2 = np.concatenate([o, g.standard_normal((1, 5, 8))])
    ls2 = np.concatenate([ls, np.full((1, 5), -np.inf)])
    a, al = oracle.merge_lse(o, ls)
    b, bl = oracle.merge_lse(o2, ls2)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
    np.testing.assert_allclose(al, bl, rtol=0, atol=1e-15)
    # order independence
    c, cl = oracle.merge_lse(o[::-1], ls[::-1])
    np.testing.assert_allclose(a, c, rtol=0, atol=1e-14)
    np.testing.assert_allclose(al, cl, rtol=0, atol=1e-14)
    # closed form with two equal parts: lse + ln 2, mean of outputs
    e, el = oracle.merge_lse(np.stack([o[0], o[1]]), np.stack([ls[0], ls[0]]))
    np.testing.assert_allclose(e, (o[0] + o[1]) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(el, ls[0] + np.log(2), rtol=0, atol=1e-15)
    # all -inf: out 0, lse -inf
    z, zl = oracle.merge_lse(o, np.full((3, 5), -np.inf))
    assert (z == 0).all() and (zl == -np.inf).all()


def test_empty_key_set():
    kp, vp, table, n_pages = indicator_case(300, 4, 11)
    Q = np.ones((1, 2, D), np.float32)
    o, l_ = oracle.decode(Q, 2, kp, vp, table, n_pages, 300, 1 / 16, blocks=np.array([[-5, 50]]))
    assert (o == 0).all() and (l_ == -np.inf).all()
