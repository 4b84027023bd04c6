"""GPU parity of the Hadamard rotation (kvattn_rotate_rows) and of a cache
built from rotated keys: rotated rows equal the oracle's binary32 butterflies
bit for bit, the pool written from rotated keys equals the oracle's bit for
bit, attention with rotated queries matches the oracle within the decode bar,
and on keys with a few large channels the rotated cache is closer to exact
(unquantised) attention than the plain one."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant, rotate
import long_context_attention_paged_amd as kv
from kvtest_util import DEV, Pools, compare, gpu, host

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3


@pytest.mark.parametrize("n_rows", [1, 3, 4, 5, 1000, 4097])
def test_rotate_rows_bitexact(n_rows):
    g = np.random.default_rng(n_rows)
    x = (g.standard_normal((n_rows, 256)) * np.exp(2 * g.standard_normal((n_rows, 1)))).astype(
        np.float32)
    x[0, :7] = [0.0, -0.0, 1e-30, 3e30, -2.5, 1.0, 7.0]  # zeros, tiny and huge entries
    d = gpu(x)
    kv.kvattn_rotate_rows(d)
    torch.cuda.synchronize()
    assert (host(d).view(np.uint32) == rotate.rotate_rows_f32(x).view(np.uint32)).all()


def outlier_kv(g, kv_len, n_kv):
    K = g.standard_normal((kv_len, n_kv, 256)).astype(np.float32)
    V = g.standard_normal((kv_len, n_kv, 256)).astype(np.float32)
    for h in range(n_kv):  # four channels x8 per head, as the decode-131k workload plants
        K[:, h, g.choice(256, 4, replace=False)] *= 8.0
    return K, V


def test_rotated_cache_parity_and_error():
    n_kv, gqa, kv_len, n_q_tok = 2, 6, 3000, 4
    g = np.random.default_rng(77)
    n_pages = (kv_len + 127) // 128
    table = g.permutation(n_pages + 2)[:n_pages].astype(np.int32)
    K, V = outlier_kv(g, kv_len, n_kv)
    q = g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32)

    # GPU: rotate the keys and the queries with the library, then the usual path
    Kd, qd = gpu(K), gpu(q)
    kv.kvattn_rotate_rows(Kd)
    kv.kvattn_rotate_rows(qd)
    rot = Pools(n_pages + 2, n_kv, gqa, init_seed=3)
    kv.kvattn_quantize_pages(rot.geom, Kd, gpu(V), 0, gpu(table, torch.int32), rot.gk, rot.gv)
    out_r, lse_r = kv.kvattn_decode(rot.geom, qd, rot.gk, rot.gv, gpu(table, torch.int32), kv_len,
                                    1 / 16)
    # oracle: the same rotation in its own code, then its quantiser and attention
    Kr = rotate.rotate_rows_f32(K)
    qr = rotate.rotate_rows_f32(q)
    quant.quantize_into_pool(Kr, V, 0, table, rot.ok, rot.ov)
    gk, gv = rot.gpu_bytes()
    assert (gk == rot.ok).all() and (gv == rot.ov).all(), "rotated pool bytes differ"
    ref_o, ref_l = oracle.decode(qr, gqa, rot.ok, rot.ov, table, n_pages, kv_len, 1 / 16)
    eo, el, rr = compare(out_r, lse_r, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)

    # the same cache without rotation
    plain = Pools(n_pages + 2, n_kv, gqa)
    plain.write(K, V, 0, table)
    out_p, _ = kv.kvattn_decode(plain.geom, gpu(q), plain.gk, plain.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16)
    # exact attention over the unquantised keys and values (binary64)
    exact = np.zeros((n_q_tok, n_kv * gqa, 256))
    pos = np.arange(kv_len)
    for h in range(n_kv):
        rows = q[:, h * gqa:(h + 1) * gqa].reshape(-1, 256)
        limits = np.repeat(kv_len - n_q_tok + np.arange(n_q_tok), gqa)
        o, _ = oracle.attend_rows(rows, K[:, h].astype(np.float64), V[:, h].astype(np.float64),
                                  pos, limits, 1 / 16)
        exact[:, h * gqa:(h + 1) * gqa] = o.reshape(n_q_tok, gqa, 256)
    # both caches quantise V the same way; the rotation only changes the key error
    err_r = np.abs(host(out_r) - exact).max()
    err_p = np.abs(host(out_p) - exact).max()
    assert err_r < err_p, (err_r, err_p)


def test_rotated_values_round_trip_through_the_output():
    """Values rotated before quantisation too: H/16 is symmetric and
    orthonormal, so rotating the attention output rows once more gives the
    attention over the unrotated values; matches the oracle's same pipeline."""
    n_kv, gqa, kv_len, n_q_tok = 1, 6, 2000, 1
    g = np.random.default_rng(78)
    n_pages = (kv_len + 127) // 128
    table = np.arange(n_pages, dtype=np.int32)
    K, V = outlier_kv(g, kv_len, n_kv)
    V[:, 0, g.choice(256, 4, replace=False)] *= 8.0
    q = g.standard_normal((n_q_tok, gqa, 256)).astype(np.float32)
    Kd, Vd, qd = gpu(K), gpu(V), gpu(q)
    for t in (Kd, Vd, qd):
        kv.kvattn_rotate_rows(t)
    pools = Pools(n_pages, n_kv, gqa)
    kv.kvattn_quantize_pages(pools.geom, Kd, Vd, 0, gpu(table, torch.int32), pools.gk, pools.gv)
    out, lse = kv.kvattn_decode(pools.geom, qd, pools.gk, pools.gv, gpu(table, torch.int32),
                                kv_len, 1 / 16)
    kv.kvattn_rotate_rows(out)
    quant.quantize_into_pool(rotate.rotate_rows_f32(K), rotate.rotate_rows_f32(V), 0, table,
                             pools.ok, pools.ov)
    gk, gv = pools.gpu_bytes()
    assert (gk == pools.ok).all() and (gv == pools.ov).all()
    ref_o, ref_l = oracle.decode(rotate.rotate_rows_f32(q), gqa, pools.ok, pools.ov, table,
                                 n_pages, kv_len, 1 / 16)
    ref_o = rotate.rotate_rows_f64(ref_o)
    eo, el, rr = compare(out, lse, ref_o, ref_l)
    assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (eo, el, rr)
