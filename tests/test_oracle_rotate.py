"""Pins of the oracle's Hadamard rotation (oracle/rotate.py) against things
other than itself: scipy's Sylvester Hadamard matrix, exact integer
arithmetic, the binary64 matrix product, and the transform's own algebra."""
import numpy as np
import pytest
import scipy.linalg

from oracle import quant, rotate


def test_matrix_is_scipys_sylvester_hadamard():
    h = rotate.hadamard_matrix(256)
    assert (h == scipy.linalg.hadamard(256)).all()
    assert (h @ h.T == 256 * np.eye(256)).all()


def test_butterflies_are_exact_on_small_integers():
    """Integer rows with |x| <= 8: every butterfly sum stays below 2^24, so the
    binary32 result times 16 is exactly H x (integer matrix product)."""
    g = np.random.default_rng(0)
    x = g.integers(-8, 9, (50, 256)).astype(np.float32)
    y = rotate.rotate_rows_f32(x)
    ref = x.astype(np.int64) @ scipy.linalg.hadamard(256).T
    assert (y.astype(np.float64) * 16 == ref).all()
    # H H = 256 I and each pass divides by 16: two passes give the row back exactly
    assert (rotate.rotate_rows_f32(y) == x).all()
    e = np.zeros((1, 256), np.float32)
    e[0, 37] = 1.0
    assert (rotate.rotate_rows_f32(e)[0] == scipy.linalg.hadamard(256)[:, 37] / 16).all()


def test_binary32_within_rounding_of_the_definition():
    """Each of the 8 butterfly stages rounds once; the sums grow at most 2x per
    stage, so the error is below 2^-24 * 256 * max|x| / 16 per element."""
    g = np.random.default_rng(1)
    x = (g.standard_normal((200, 256)) * np.exp(g.standard_normal((200, 1)))).astype(np.float32)
    y = rotate.rotate_rows_f32(x).astype(np.float64)
    ref = rotate.rotate_rows_f64(x)
    bound = 2.0 ** -24 * 256 / 16 * np.abs(x).max(axis=1, keepdims=True)
    assert (np.abs(y - ref) <= bound).all()
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1),
                               rtol=1e-6)


def test_rotation_keeps_dot_products_and_lowers_q8_0_error_on_outliers():
    """(H q/16).(H k/16) = q.k, and on keys with a few large channels (the
    decode workload's x8 outliers) the rotated keys quantise with less error."""
    g = np.random.default_rng(2)
    k = g.standard_normal((512, 256)).astype(np.float32)
    k[:, [3, 70, 141, 200]] *= 8.0
    q = g.standard_normal((4, 256)).astype(np.float32)
    kr, qr = rotate.rotate_rows_f64(k), rotate.rotate_rows_f64(q)
    np.testing.assert_allclose(qr @ kr.T, q.astype(np.float64) @ k.T.astype(np.float64),
                               rtol=1e-9, atol=1e-9)

    def q8_roundtrip(rows):
        codes, d = quant.q8_0_quantize(np.asarray(rows, np.float32).reshape(-1, 8, 32))
        return quant.q8_0_dequantize(codes, d).reshape(rows.shape)

    plain = q8_roundtrip(k)
    rot = rotate.rotate_rows_f64(q8_roundtrip(rotate.rotate_rows_f32(k)))  # back to k's basis
    err_plain = np.sqrt(((plain - k) ** 2).mean())
    err_rot = np.sqrt(((rot - k) ** 2).mean())
    assert err_rot < 0.6 * err_plain, (err_rot, err_plain)
