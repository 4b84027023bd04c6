"""Pins for the oracle's quantisation, page layout and block summaries.

Each test checks the oracle against something other than itself: sizes the
pages print (tests/golden/page_figures.json), IEEE-754 facts, closed forms,
round-trip bounds, idempotence, and a hand-built layout word.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import quant

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_record_sizes_match_page_figures():
    """Block sizes reproduce the pages' per-token byte counts.
    [VULKAN] 模型結構: 16 layers x 4 KV heads x 256 = 16384 elements per token;
    f16 K+V at 64K tokens = 4 GiB. [VULKAN] 坑 2: q4_0 K+V = 18 KiB/token.
    [VULKAN] closing remark: q8_0 K = 8.5 bits per element."""
    elems = GOLD["elements_per_token_per_kv"]["value"]
    assert 16 * 4 * quant.HEAD_DIM == elems
    assert elems * 2 * 2 * 65536 == GOLD["f16_bytes_per_64k_tokens"]["value"]
    q8_block = quant.K_RECORD_BYTES // (quant.PAGE_TOKENS * quant.N_BLOCKS)
    q4_block = quant.V_RECORD_BYTES // (quant.PAGE_TOKENS * quant.N_BLOCKS)
    assert q8_block == 34 and q4_block == 18
    assert q8_block * 8 / 32 == GOLD["q8_0_bits_per_element"]["value"]
    assert elems * 2 * q4_block // 32 == GOLD["q4_0_kv_bytes_per_token"]["value"]
    # this build's Q8_0 K + Q4_0 V: 26 KiB per token over the 16 x 4 x 256 shape
    assert elems * (q8_block + q4_block) // 32 == 26 * 1024
    assert quant.PAGE_TOKENS == GOLD["kvmem_block_tokens"]["value"]


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -11, 1.0),                 # exact tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),  # exact tie -> even
    (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),  # above the tie
    (2049.0, 2048.0),
    (2051.0, 2052.0),
    (65504.0, 65504.0),
    (65519.0, 65504.0),
    (65520.0, np.inf),                        # tie at the overflow threshold
    (2.0 ** -24, 2.0 ** -24),                 # smallest subnormal
    (2.0 ** -25, 0.0),                        # tie between 0 and 2^-24 -> even (0)
    (3 * 2.0 ** -26, 2.0 ** -24),
])
def test_rn16_ieee_facts(x, expect):
    assert float(quant.rn16(np.float32(x))) == expect


def _f16_finite_nonneg():
    """Every non-negative finite binary16 value, ascending (bit patterns
    0x0000 .. 0x7BFF decoded exactly), as binary64."""
    return np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_rn16_every_midpoint_and_neighbours():
    """Exhaustive round-to-nearest-even to binary16: for every pair of
    adjacent finite binary16 values a < b (both signs), the binary32 midpoint
    (exact: it needs 12 significant bits) rounds to the one whose bit pattern
    is even, and the binary32 numbers just below and just above it round to a
    and to b. The top midpoint 65520 overflows to infinity (its even
    neighbour 65536 is out of range) and the number below it gives 65504."""
    v = _f16_finite_nonneg()
    a, b = v[:-1], v[1:]
    mid = ((a + b) / 2).astype(np.float32)
    assert (mid.astype(np.float64) == (a + b) / 2).all()          # midpoints exact
    even_is_a = (np.arange(len(a)) % 2) == 0                      # bit pattern of a even
    want = np.where(even_is_a, a, b)
    below = np.nextafter(mid, np.float32(-np.inf))
    above = np.nextafter(mid, np.float32(np.inf))
    for sign in (1.0, -1.0):
        s32 = np.float32(sign)
        assert (quant.rn16(s32 * mid).astype(np.float64) == sign * want).all()
        assert (quant.rn16(s32 * below).astype(np.float64) == sign * a).all()
        assert (quant.rn16(s32 * above).astype(np.float64) == sign * b).all()
    top = np.float32(65520.0)
    assert quant.rn16(top) == np.inf and quant.rn16(-top) == -np.inf
    assert quant.rn16(np.nextafter(top, np.float32(0))) == 65504.0
    # every binary16 value is a fixed point
    assert (quant.rn16(v.astype(np.float32)).astype(np.float64) == v).all()


def test_code_rounding_ties_go_to_even():
    """Code rounding is rint, half to even (include/kvattn.h): hand-built
    blocks whose products x * inv land exactly on k + 1/2. Rounding half away
    from zero would give the codes in the comments instead."""
    # Q8_0 with amax 127 -> d = 1, inv = 1
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]
    c, b = quant.q8_0_quantize(x)
    assert quant.f16_from_bits(b) == 1.0
    assert list(c[1:9]) == [2, 4, -2, -4, 0, 0, 2, 126]   # away: 3, 4, -3, -4, 1, -1, 2, 127
    # Q4_0 with the extreme -8 at index 0 -> d = 1, inv = 1; code = rint(x) + 8
    x = np.zeros(32, np.float32)
    x[0] = -8.0
    x[1:8] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 6.5]
    c, b = quant.q4_0_quantize(x)
    assert quant.f16_from_bits(b) == 1.0 and c[0] == 0
    assert list(c[1:8]) == [10, 12, 6, 4, 8, 8, 14]       # away: 11, 12, 5, 4, 9, 7, 15
    # Q5_1 with min 0 and max 31 -> d = 1, m = 0, inv = 1; code = rint(x)
    x = np.zeros(32, np.float32)
    x[31] = 31.0
    x[1:7] = [2.5, 3.5, 10.5, 11.5, 0.5, 30.5]
    c, db, mb = quant.q5_1_quantize(x)
    assert quant.f16_from_bits(db) == 1.0 and quant.f16_from_bits(mb) == 0.0
    assert list(c[1:7]) == [2, 4, 10, 12, 0, 30]          # away: 3, 4, 11, 12, 1, 31


def test_q5_1_codes_use_the_stored_minimum():
    """Q5_1 codes are taken from x - m with m the STORED binary16 minimum
    (include/kvattn.h): block minimum 0.1f, which binary16 stores as
    0.0999755859375 (bits 0x2E66), maximum 1.06875f, so d = RN16(0.96875 / 31)
    = 2^-5 and inv = 32. For x = 0.42810997f, (x - m) * 32 = 10.5003 gives
    code 11; the unrounded minimum would give 10.4995 and code 10."""
    mn, mx, x5 = np.float32(0.1), np.float32(1.06875), np.float32(0.42810997)
    blk = np.linspace(mn, mx, 32).astype(np.float32)
    blk[0], blk[31], blk[5] = mn, mx, x5
    c, db, mb = quant.q5_1_quantize(blk)
    assert mb == 0x2E66 and quant.f16_from_bits(mb) == np.float32(0.0999755859375)
    assert quant.f16_from_bits(db) == np.float32(2.0 ** -5)
    assert c[5] == 11
    assert c[0] == 0 and c[31] == 31


def test_q8_0_closed_forms():
    # zero block: codes 0, scale +0 (bits 0x0000)
    c, b = quant.q8_0_quantize(np.zeros(32, np.float32))
    assert (c == 0).all() and b == 0
    # x_i = k_i * d with d = 2^-7 and max |k| = 127: exact round trip
    g = np.random.default_rng(1)
    k = g.integers(-127, 128, 32)
    k[5] = -127
    x = (k * 2.0 ** -7).astype(np.float32)
    c, b = quant.q8_0_quantize(x)
    assert (c == k).all() and quant.f16_from_bits(b) == 2.0 ** -7
    # one-hot: the hot element gets code +-127, the rest 0
    x = np.zeros(32, np.float32)
    x[9] = -3.0
    c, b = quant.q8_0_quantize(x)
    assert c[9] == -127 and (np.delete(c, 9) == 0).all()
    assert quant.f16_from_bits(b) == quant.rn16(np.float32(3.0) / np.float32(127.0))
    # constant block: every code 127
    c, _ = quant.q8_0_quantize(np.full(32, 0.37, np.float32))
    assert (c == 127).all()


def test_q4_0_closed_forms():
    # zero block: every code 8 and scale +0
    c, b = quant.q4_0_quantize(np.zeros(32, np.float32))
    assert (c == 8).all() and b == 0
    # constant block c: the signed extreme maps to code 0, d = -c/8, xhat = c exactly
    for val in (0.5, -4.0):
        c, b = quant.q4_0_quantize(np.full(32, val, np.float32))
        assert (c == 0).all()
        assert quant.f16_from_bits(b) == -val / 8
        assert (quant.q4_0_dequantize(c, b) == val).all()
    # exact grid: x = k*d, k in [-8, 7], unique extreme k=-8 at index 3
    g = np.random.default_rng(2)
    k = g.integers(-7, 8, 32)
    k[3] = -8
    x = (k * 2.0 ** -5).astype(np.float32)
    c, b = quant.q4_0_quantize(x)
    assert (c.astype(int) - 8 == k).all() and quant.f16_from_bits(b) == 2.0 ** -5
    # magnitude tie: the LOWEST index sets the sign of the scale
    x = np.zeros(32, np.float32)
    x[3], x[7] = 1.0, -1.0
    c, b = quant.q4_0_quantize(x)
    assert quant.f16_from_bits(b) == -0.125 and c[3] == 0 and c[7] == 15
    x[3], x[7] = -1.0, 1.0
    c, b = quant.q4_0_quantize(x)
    assert quant.f16_from_bits(b) == 0.125 and c[3] == 0 and c[7] == 15
    # scale underflow in binary16: stored as +0, codes 8
    x = np.zeros(32, np.float32)
    x[0] = 1e-9
    c, b = quant.q4_0_quantize(x)
    assert b == 0 and (c == 8).all()


def _random_blocks(n, seed, outlier=False):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, 32)).astype(np.float32)
    x[: n // 4] *= np.float32(8.0)
    x[n // 4: n // 2] *= np.float32(1e-3)
    if outlier:
        x[:, 7] *= np.float32(50.0)
    return x


@pytest.mark.parametrize("seed", [0, 1])
def test_roundtrip_bounds(seed):
    """|x - xhat| <= d/2 (plus binary32 product rounding) for Q8_0;
    <= |d|/2 for unclamped Q4_0 codes. On the clamped +7 side |x| <= |m| and
    binary16 rounding gives |d| >= |m|/8 * (1 - 2^-11), so
    |x - xhat| <= |d| * (8 / (1 - 2^-11) - 7)."""
    x = _random_blocks(4096, seed, outlier=bool(seed))
    c, b = quant.q8_0_quantize(x)
    d = quant.f16_from_bits(b).astype(np.float64)
    err = np.abs(x - quant.q8_0_dequantize(c, b))
    assert (err <= d[:, None] * (0.5 + 2.0 ** -14)).all()
    c, b = quant.q4_0_quantize(x)
    d = np.abs(quant.f16_from_bits(b).astype(np.float64))
    err = np.abs(x - quant.q4_0_dequantize(c, b))
    clamped = c == 15
    assert (err[~clamped] <= np.broadcast_to(d[:, None], x.shape)[~clamped] * (0.5 + 2.0 ** -14)).all()
    assert (err <= d[:, None] * (8.0 / (1.0 - 2.0 ** -11) - 7.0 + 2.0 ** -14)).all()
    # every Q4_0 block uses code 0 for its signed extreme
    assert (c.min(axis=1) == 0).all()


@pytest.mark.parametrize("seed", [3, 4])
def test_idempotence(seed):
    x = _random_blocks(4096, seed)
    c, b = quant.q8_0_quantize(x)
    c2, b2 = quant.q8_0_quantize(quant.q8_0_dequantize(c, b).astype(np.float32))
    assert (c == c2).all() and (b == b2).all()
    c, b = quant.q4_0_quantize(x)
    c2, b2 = quant.q4_0_quantize(quant.q4_0_dequantize(c, b).astype(np.float32))
    assert (c == c2).all() and (b == b2).all()


def test_pack_unpack_roundtrip():
    g = np.random.default_rng(5)
    kc = g.integers(-127, 128, (3, 128, 256)).astype(np.int8)
    kb = g.integers(0, 65536, (3, 128, 8)).astype(np.uint16)
    vc = g.integers(0, 16, (3, 128, 256)).astype(np.uint8)
    vb = g.integers(0, 65536, (3, 128, 8)).astype(np.uint16)
    rk = quant.pack_k_record(kc, kb)
    rv = quant.pack_v_record(vc, vb)
    assert rk.shape == (3, quant.K_RECORD_BYTES) and rv.shape == (3, quant.V_RECORD_BYTES)
    kc2, kb2 = quant.unpack_k_record(rk)
    vc2, vb2 = quant.unpack_v_record(rv)
    assert (kc2 == kc).all() and (kb2 == kb).all() and (vc2 == vc).all() and (vb2 == vb).all()


def test_layout_words_by_hand():
    """Hand-built bytes for the layout written in include/kvattn.h.
    K: code (t, n) at t*256 + n; scale (t, b) at 32768 + 2*(t*8 + b).
    V word w = (((c*4+q)*4+g)*16+d)*4+e holds dim 16*(4q+e)+d for slots
    32c + 16*(j//4) + 4g + j%4, slot j at bit 4*(j//2) + 16*(j%2)."""
    kc = np.zeros((128, 256), np.int8)
    kb = np.zeros((128, 8), np.uint16)
    kc[5, 200] = -3
    kb[5, 6] = 0x3C00
    rk = quant.pack_k_record(kc, kb)
    assert rk[5 * 256 + 200] == 0xFD
    assert rk[32768 + 2 * (5 * 8 + 6)] == 0x00 and rk[32768 + 2 * (5 * 8 + 6) + 1] == 0x3C
    assert rk.sum() == 0xFD + 0x3C
    # V: word with c=1, q=2, g=3, d=5, e=1 -> dim 16*(8+1)+5 = 149;
    # slots j=0..7 -> tokens 32+12+{0,1,2,3} and 32+16+12+{0,1,2,3}
    vc = np.full((128, 256), 0, np.uint8)
    toks = [44, 45, 46, 47, 60, 61, 62, 63]
    for j, t in enumerate(toks):
        vc[t, 149] = j + 1                      # codes 1..8
    vb = np.zeros((128, 8), np.uint16)
    vb[61, 4] = 0xABCD                          # slot j=5 of (c=1, g=3), block 4
    rv = quant.pack_v_record(vc, vb)
    w = (((1 * 4 + 2) * 4 + 3) * 16 + 5) * 4 + 1
    word = int.from_bytes(rv[4 * w: 4 * w + 4].tobytes(), "little")
    expect = 0
    for j in range(8):
        expect |= (j + 1) << (4 * (j // 2) + 16 * (j % 2))
    assert word == expect == 0x86427531
    others = np.frombuffer(rv[:16384].tobytes(), "<u4").copy()
    others[w] = 0
    assert (others == 0).all()
    si = ((1 * 8 + 4) * 4 + 3) * 8 + 5
    assert rv[16384 + 2 * si] == 0xCD and rv[16384 + 2 * si + 1] == 0xAB
    assert rv[16384:].astype(int).sum() == 0xCD + 0xAB


def test_quantize_into_pool_partial_and_skip():
    """Writes land in the right slots through the page table, untouched bytes
    survive, and an out-of-range page-table entry is skipped."""
    g = np.random.default_rng(6)
    n_kv, n_phys = 2, 5
    kp = g.integers(0, 256, (n_phys, n_kv, quant.K_RECORD_BYTES)).astype(np.uint8)
    vp = g.integers(0, 256, (n_phys, n_kv, quant.V_RECORD_BYTES)).astype(np.uint8)
    kp0, vp0 = kp.copy(), vp.copy()
    table = np.array([3, 0, 4, 99], np.int32)   # logical page 3 maps outside the pool
    pos0, n = 100, 300                          # positions 100..399: pages 0,1,2,3
    K = g.standard_normal((n, n_kv, 256)).astype(np.float32)
    V = g.standard_normal((n, n_kv, 256)).astype(np.float32)
    quant.quantize_into_pool(K, V, pos0, table, kp, vp)
    assert (kp[[1, 2]] == kp0[[1, 2]]).all() and (vp[[1, 2]] == vp0[[1, 2]]).all()
    for h in range(n_kv):
        for pos in (100, 127, 128, 255, 256, 383):
            lp, t = pos // 128, pos % 128
            c, b = quant.unpack_k_record(kp[table[lp], h])
            cq, bq = quant.q8_0_quantize(K[pos - pos0, h].reshape(8, 32))
            assert (c[t] == cq.reshape(-1)).all() and (b[t] == bq).all()
            c, b = quant.unpack_v_record(vp[table[lp], h])
            cq, bq = quant.q4_0_quantize(V[pos - pos0, h].reshape(8, 32))
            assert (c[t] == cq.reshape(-1)).all() and (b[t] == bq).all()
        # slot 99 of logical page 0 (physical 3) was not written
        c, b = quant.unpack_k_record(kp[3, h])
        c0, b0 = quant.unpack_k_record(kp0[3, h])
        assert (c[:100] == c0[:100]).all() and (b[:100] == b0[:100]).all()
        c, b = quant.unpack_v_record(vp[3, h])
        c0, b0 = quant.unpack_v_record(vp0[3, h])
        assert (c[:100] == c0[:100]).all() and (b[:100] == b0[:100]).all()


def test_page_summary_closed_forms():
    # every key in a page equal to a constant grid vector -> summary equals it exactly
    vec = (np.arange(256) % 17 - 8).astype(np.float32) * np.float32(0.25)
    codes, bits = quant.q8_0_quantize(np.tile(vec, (128, 1)).reshape(128, 8, 32))
    rec = quant.pack_k_record(codes.reshape(128, 256), bits)
    khat = quant.q8_0_dequantize(codes, bits).reshape(128, 256)
    assert (quant.page_summary(rec) == khat[0].astype(np.float32)).all()
    # alternating +a / -a keys sum to zero exactly
    codes = np.zeros((128, 256), np.int8)
    codes[0::2] = 100
    codes[1::2] = -100
    bits = np.full((128, 8), 0x3C00, np.uint16)
    assert (quant.page_summary(quant.pack_k_record(codes, bits)) == 0).all()
    # one token with code 128*... : summary = d * c / 128 exactly
    codes = np.zeros((128, 256), np.int8)
    codes[17, 3] = 64
    s = quant.page_summary(quant.pack_k_record(codes, bits))
    assert s[3] == 0.5 and (np.delete(s, 3) == 0).all()


def test_q8_value_record_layout_positions():
    """Q8_0 value records: bytes at hand-computed positions of the layout in
    include/kvattn.h (byte c*8192 + q*1024 + (16g + r16)*16 + 8*half + j holds
    dim 32q + 16*half + r16 of slot 32c + 16*(j//4) + 4g + j%4), 272 bytes per
    token and head (8.5 bits per element, as for keys), and a round trip."""
    assert quant.V8_RECORD_BYTES == 34816 and quant.V8_RECORD_BYTES // 128 == 272
    codes = np.zeros((128, 256), np.int8)
    bits = np.zeros((128, 8), np.uint16)
    marks = {  # (slot, dim) -> expected byte offset
        (0, 0): 0, (1, 0): 1, (16, 0): 4, (4, 0): 256, (0, 16): 8, (0, 1): 16,
        (0, 32): 1024, (32, 0): 8192, (127, 255): 3 * 8192 + 7 * 1024 + (16 * 3 + 15) * 16 + 8 + 7,
    }
    for n, (t, d) in enumerate(marks):
        codes[t, d] = n + 1
    rec = quant.pack_v8_record(codes, bits)
    for n, ((t, d), off) in enumerate(marks.items()):
        assert rec[off] == n + 1, (t, d, off)
    assert int((rec[:32768] != 0).sum()) == len(marks)
    g = np.random.default_rng(8)
    c2 = g.integers(-127, 128, (3, 128, 256)).astype(np.int8)
    b2 = g.integers(0, 1 << 16, (3, 128, 8)).astype(np.uint16)
    c3, b3 = quant.unpack_v8_record(quant.pack_v8_record(c2, b2))
    assert (c3 == c2).all() and (b3 == b2).all()
    # scales follow the Q4_0 value record's scale order
    r4 = quant.pack_v_record(np.zeros((128, 256), np.uint8), b2[0])
    r8 = quant.pack_v8_record(np.zeros((128, 256), np.int8), b2[0])
    assert (r4[16384:] == r8[32768:]).all()


def test_q8_values_quantise_like_keys():
    """With a Q8_0 value pool the values go through the key rule: the pool's
    dequantised values equal the dequantised keys of the same numbers."""
    g = np.random.default_rng(9)
    n_tok, n_kv = 300, 2
    x = g.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    x[5, 0, :32] = 0.0
    table = np.array([2, 0, 3], np.int32)
    kp = np.zeros((4, n_kv, quant.K_RECORD_BYTES), np.uint8)
    vp = np.zeros((4, n_kv, quant.V8_RECORD_BYTES), np.uint8)
    quant.quantize_into_pool(x, x, 0, table, kp, vp)
    kh, vh = oracle.dequant_page(kp[table], vp[table])
    assert (kh == vh).all()
    assert not (vh == 0).all()


def test_q4_key_record_layout_positions():
    """Q4_0 key records: nibbles at hand-computed positions of the layout in
    include/kvattn.h (slot t's row of 32 words at byte t*128; dim 8w + k in
    word w at bit 4(k/2) + 16(k%2)), 144 bytes per token and head (4.5 bits
    per element, so q4_0 K + V is 288 bytes: 18 KiB per token at 16 layers
    x 4 KV heads), scales in the Q8_0 key order, and a round trip."""
    assert quant.K4_RECORD_BYTES == 18432 and quant.K4_RECORD_BYTES // 128 == 144
    assert (144 + 144) * 16 * 4 == 18 * 1024
    codes = np.zeros((128, 256), np.uint8)
    bits = np.zeros((128, 8), np.uint16)
    marks = {  # (slot, dim) -> (byte offset, shift inside the byte)
        (0, 0): (0, 0), (0, 1): (2, 0), (0, 2): (0, 4), (0, 3): (2, 4), (0, 4): (1, 0),
        (0, 7): (3, 4), (0, 8): (4, 0), (1, 0): (128, 0), (127, 255): (127 * 128 + 127, 4),
    }
    for n, (t, d) in enumerate(marks):
        codes[t, d] = n + 1
    rec = quant.pack_k4_record(codes, bits)
    for n, ((t, d), (off, sh)) in enumerate(marks.items()):
        assert (rec[off] >> sh) & 0xF == n + 1, (t, d, off, sh)
    nib = np.stack([rec[:16384] & 0xF, rec[:16384] >> 4])
    assert int(np.count_nonzero(nib)) == len(marks)      # nothing else written
    g = np.random.default_rng(10)
    c2 = g.integers(0, 16, (3, 128, 256)).astype(np.uint8)
    b2 = g.integers(0, 1 << 16, (3, 128, 8)).astype(np.uint16)
    c3, b3 = quant.unpack_k4_record(quant.pack_k4_record(c2, b2))
    assert (c3 == c2).all() and (b3 == b2).all()
    r8 = quant.pack_k_record(np.zeros((128, 256), np.int8), b2[0])
    r4 = quant.pack_k4_record(np.zeros((128, 256), np.uint8), b2[0])
    assert (r8[32768:] == r4[16384:]).all()


def test_q4_keys_quantise_like_values():
    """With a Q4_0 key pool the keys go through the Q4_0 value rule: the
    pool's dequantised keys equal the dequantised values of the same numbers,
    and a full page's summary is the binary64 mean of those keys."""
    g = np.random.default_rng(11)
    n_tok, n_kv = 300, 2
    x = g.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    x[5, 0, :32] = 0.0
    x[6, 1, 32:64] = 0.5
    x[6, 1, 40], x[6, 1, 50] = -2.0, 2.0                # tie: the lower index sets the sign
    table = np.array([2, 0, 3], np.int32)
    kp = np.zeros((4, n_kv, quant.K4_RECORD_BYTES), np.uint8)
    vp = np.zeros((4, n_kv, quant.V_RECORD_BYTES), np.uint8)
    quant.quantize_into_pool(x, x, 0, table, kp, vp)
    kh, vh = oracle.dequant_page(kp[table], vp[table])
    assert (kh == vh).all()
    assert kh[0, 1, 6, 40] == -2.0 and kh[0, 1, 6, 50] == 2.0 * 7 / 8
    s = quant.summaries_from_pool(kp, table, 2, n_kv)
    for p in range(2):
        for h in range(n_kv):
            exact = np.float32(np.sum(kh[p, h], axis=0, dtype=np.float64) / 128.0)
            assert np.abs(s[h, p] - exact).max() <= 1e-7 * (1 + np.abs(exact).max())


def test_q5_1_rule_closed_forms():
    """Q5_1: a block on an exact grid m + d*k keeps its codes and values; a
    constant block has scale 0 and dequantises to RN16 of the constant; any
    block dequantises within d/2 plus the binary16 rounding of m."""
    d, m = 0.125, -1.5                                    # both exact in binary16
    k = np.arange(32)
    x = (m + d * k).astype(np.float32)[::-1].copy()       # order does not matter
    codes, db, mb = quant.q5_1_quantize(x)
    assert (codes == k[::-1]).all()
    assert quant.f16_from_bits(db) == np.float32(d) and quant.f16_from_bits(mb) == np.float32(m)
    assert (quant.q5_1_dequantize(codes, db, mb) == x).all()
    c = np.full(32, 0.3, np.float32)
    codes, db, mb = quant.q5_1_quantize(c)
    assert db == 0 and (codes == 0).all()
    assert (quant.q5_1_dequantize(codes, db, mb) == np.float32(np.float16(0.3))).all()
    g = np.random.default_rng(12)
    x = (g.standard_normal((500, 32)) * np.exp(g.standard_normal((500, 1)))).astype(np.float32)
    codes, db, mb = quant.q5_1_quantize(x)
    dq = quant.q5_1_dequantize(codes, db, mb)
    dd = quant.f16_from_bits(db).astype(np.float64)
    mm = quant.f16_from_bits(mb).astype(np.float64)
    bound = dd / 2 * (1 + 1e-3) + np.abs(mm - x.min(axis=1)) + 1e-12
    assert (np.abs(dq - x).max(axis=1) <= bound + dd * 1e-3).all()
    assert codes.max() == 31 and codes.min() == 0


def test_q5_1_key_record_layout_positions():
    """Q5_1 key records: low nibbles where a Q4_0 key record puts them, the
    fifth bits at hand-computed bit positions (byte 16384 + t*32 + w, dim
    8w + 2p at bit p, 8w + 2p + 1 at bit 4 + p), d at 20480 + 2(t*8 + b), m at
    22528 + 2(t*8 + b); 192 bytes per token and head (6 bits per element);
    a round trip."""
    assert quant.K5_RECORD_BYTES == 24576 and quant.K5_RECORD_BYTES // 128 == 192
    codes = np.zeros((128, 256), np.uint8)
    z = np.zeros((128, 8), np.uint16)
    marks = {(0, 0): (16384, 0), (0, 1): (16384, 4), (0, 2): (16384, 1), (0, 7): (16384, 7),
             (0, 8): (16385, 0), (3, 255): (16384 + 3 * 32 + 31, 7)}
    for (t, dm) in marks:
        codes[t, dm] = 16                                # only the fifth bit set
    rec = quant.pack_k5_record(codes, z, z)
    assert not rec[:16384].any()
    for (t, dm), (off, bit) in marks.items():
        assert (rec[off] >> bit) & 1 == 1, (t, dm)
    assert int(np.unpackbits(rec[16384:20480]).sum()) == len(marks)
    db = np.zeros((128, 8), np.uint16)
    mb = np.zeros((128, 8), np.uint16)
    db[5, 3], mb[5, 3] = 0x1234, 0xABCD
    rec = quant.pack_k5_record(np.zeros((128, 256), np.uint8), db, mb)
    o = 2 * (5 * 8 + 3)
    assert rec[20480 + o] == 0x34 and rec[20481 + o] == 0x12
    assert rec[22528 + o] == 0xCD and rec[22529 + o] == 0xAB
    c4 = np.random.default_rng(13).integers(0, 16, (128, 256)).astype(np.uint8)
    r4 = quant.pack_k4_record(c4, z)
    r5 = quant.pack_k5_record(c4, z, z)
    assert (r4[:16384] == r5[:16384]).all()
    g = np.random.default_rng(14)
    c2 = g.integers(0, 32, (2, 128, 256)).astype(np.uint8)
    d2 = g.integers(0, 1 << 16, (2, 128, 8)).astype(np.uint16)
    m2 = g.integers(0, 1 << 16, (2, 128, 8)).astype(np.uint16)
    c3, d3, m3 = quant.unpack_k5_record(quant.pack_k5_record(c2, d2, m2))
    assert (c3 == c2).all() and (d3 == d2).all() and (m3 == m2).all()


def test_q5_1_keys_in_pool_and_summary():
    """A Q5_1 key pool holds the rule's codes; the summary of a full page is
    the binary64 mean of d*code + m."""
    g = np.random.default_rng(15)
    n_tok, n_kv = 260, 2
    x = g.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    x[3, 1, 64:96] = 2.0
    table = np.array([1, 2, 0], np.int32)
    kp = np.zeros((3, n_kv, quant.K5_RECORD_BYTES), np.uint8)
    vp = np.zeros((3, n_kv, quant.V_RECORD_BYTES), np.uint8)
    quant.quantize_into_pool(x, x, 0, table, kp, vp)
    codes, db, mb = quant.q5_1_quantize(x.reshape(n_tok, n_kv, 8, 32))
    kh, _ = oracle.dequant_page(kp[table], vp[table])
    ref = quant.q5_1_dequantize(codes, db, mb).reshape(n_tok, n_kv, 256)
    assert (kh[0].transpose(1, 0, 2) == ref[:128]).all()
    assert (kh[2, :, :4].transpose(1, 0, 2) == ref[256:260]).all()
    assert (kh[0, 1, 3, 64:96] == np.float64(np.float16(2.0))).all()
    s = quant.summaries_from_pool(kp, table, 2, n_kv)
    for p in range(2):
        exact = (np.sum(ref[128 * p:128 * (p + 1)], axis=0) / 128.0).astype(np.float32)
        assert (s[:, p] == exact).all()
