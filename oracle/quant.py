"""Oracle: Q8_0 / Q4_0 block quantisation, the page byte layout, and block
summaries. Test infrastructure only (see the package docstring).

The pages name the two cache types and their sizes but define neither the
scale rule nor the rounding:
  - keys Q8_0, values Q4_0: [STREAM] step ④ (-ctk q8_0 -ctv q4_0) and
    [RDNA4] opening paragraph (Q8_0/Q4_0 KV cache);
  - q8_0 K is 8.5 bits per element: [VULKAN] closing remark on K precision;
  - q4_0 K+V is 18 KiB per token at 16 layers x 4 KV heads x 256:
    [VULKAN] "坑 2" together with "模型結構".
The definitions used (amax/127 for Q8_0; signed max-magnitude element mapped
to -8 for Q4_0; every rounding IEEE round-to-nearest-even; codes computed with
the stored binary16 scale) are this build's reading and are written out in
include/kvattn.h next to the ABI they define.
"""
import numpy as np

HEAD_DIM = 256
PAGE_TOKENS = 128
BLOCK = 32
N_BLOCKS = HEAD_DIM // BLOCK
K_CODES_BYTES = PAGE_TOKENS * HEAD_DIM          # 32768
K_RECORD_BYTES = K_CODES_BYTES + PAGE_TOKENS * N_BLOCKS * 2   # 34816
V_CODES_BYTES = PAGE_TOKENS * HEAD_DIM // 2     # 16384
V_RECORD_BYTES = V_CODES_BYTES + PAGE_TOKENS * N_BLOCKS * 2   # 18432
# Q8_0 values (the q8_0/q8_0 pair, [KVMEM] 測試口徑 --kv-dtype q8_0): a value
# record of the key record's size, selected by the record size of the pool.
V8_CODES_BYTES = PAGE_TOKENS * HEAD_DIM         # 32768
V8_RECORD_BYTES = V8_CODES_BYTES + PAGE_TOKENS * N_BLOCKS * 2  # 34816
# Q4_0 keys (the q4_0/q4_0 pair of [VULKAN] "坑 2": 18 KiB per token for K+V
# at 16 layers x 4 KV heads x 256): a key record of the Q4_0 value record's
# size, selected by the record size of the key pool.
K4_CODES_BYTES = PAGE_TOKENS * HEAD_DIM // 2    # 16384
K4_RECORD_BYTES = K4_CODES_BYTES + PAGE_TOKENS * N_BLOCKS * 2  # 18432
# Q5_1 keys (the q5_1/q4_0 pair, [VULKAN] 坑 3's allowed type list; q5_1 is 6
# bits per element, [VULKAN] 坑 2): low nibbles as in the Q4_0 key record, then
# one byte of fifth bits per 8 dims, then the scales d, then the minimums m.
K5_HI_OFF = K4_CODES_BYTES                              # 16384
K5_D_OFF = K5_HI_OFF + PAGE_TOKENS * HEAD_DIM // 8      # 20480
K5_M_OFF = K5_D_OFF + PAGE_TOKENS * N_BLOCKS * 2        # 22528
K5_RECORD_BYTES = K5_M_OFF + PAGE_TOKENS * N_BLOCKS * 2  # 24576


def rn16(x):
    """Round binary32 values to the nearest binary16 (ties to even) and return
    them as binary32. numpy's float32->float16 cast is IEEE round-to-nearest-
    even, overflowing to infinity."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def f16_bits(x):
    """binary16 bit patterns (uint16) of binary32 values rounded to nearest-even."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_from_bits(bits):
    """binary32 values of binary16 bit patterns."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def q8_0_quantize(x):
    """Q8_0 of 32-element blocks along the last axis (keys).

    x: float32 [..., 32]. Returns (codes int8 [..., 32], scale_bits uint16 [...]).
    amax = max|x|; d = RN16(RN32(amax / 127)); d == 0 -> codes 0, scale +0;
    else inv = RN32(1/d), code = clamp(rint(RN32(x*inv)), -127, 127).
    """
    x = np.asarray(x, np.float32)
    assert x.shape[-1] == BLOCK
    amax = np.max(np.abs(x), axis=-1)
    d32 = amax / np.float32(127.0)                 # binary32 division, RN
    d16 = rn16(d32)
    zero = d16 == 0
    d_safe = np.where(zero, np.float32(1.0), d16)
    inv = np.float32(1.0) / d_safe                 # RN32(1/d)
    prod = x * inv[..., None]                      # RN32(x*inv)
    codes = np.clip(np.rint(prod), -127, 127)
    codes = np.where(zero[..., None], 0, codes).astype(np.int8)
    bits = np.where(zero, np.uint16(0), f16_bits(d16)).astype(np.uint16)
    return codes, bits


def q8_0_dequantize(codes, scale_bits):
    """Dequantised Q8_0 block values d*code, exact in binary64."""
    d = f16_from_bits(scale_bits).astype(np.float64)
    return np.asarray(codes, np.float64) * d[..., None]


def q4_0_quantize(x):
    """Q4_0 of 32-element blocks along the last axis (values).

    x: float32 [..., 32]. Returns (codes uint8 in [0,15] [..., 32], scale_bits).
    j* = lowest index with |x_j*| = amax, m = x_j*, d = RN16(RN32(-m/8)).
    amax == 0 or d == 0 -> scale +0 and every code 8; else inv = RN32(1/d),
    code = clamp(rint(RN32(x*inv)), -8, 7) + 8. The signed extreme maps to
    code 0 (value -8*d), so all 16 codes are used ("offset 8").
    """
    x = np.asarray(x, np.float32)
    assert x.shape[-1] == BLOCK
    ax = np.abs(x)
    jstar = np.argmax(ax, axis=-1)                 # argmax returns the lowest index
    m = np.take_along_axis(x, jstar[..., None], axis=-1)[..., 0]
    amax = np.take_along_axis(ax, jstar[..., None], axis=-1)[..., 0]
    d32 = (-m) / np.float32(8.0)
    d16 = rn16(d32)
    zero = (amax == 0) | (d16 == 0)
    d_safe = np.where(zero, np.float32(1.0), d16)
    inv = np.float32(1.0) / d_safe
    prod = x * inv[..., None]
    codes = np.clip(np.rint(prod), -8, 7) + 8
    codes = np.where(zero[..., None], 8, codes).astype(np.uint8)
    bits = np.where(zero, np.uint16(0), f16_bits(d16)).astype(np.uint16)
    return codes, bits


def q5_1_quantize(x):
    """Q5_1 of 32-element blocks along the last axis (keys of the q5_1 pair).

    x: float32 [..., 32]. Returns (codes uint8 in [0,31] [..., 32], d_bits,
    m_bits). mn = min x, mx = max x; d = RN16(RN32((mx - mn) / 31)),
    m = RN16(mn). d == 0 -> scale +0 and every code 0; else inv = RN32(1/d),
    code = clamp(rint(RN32(RN32(x - m) * inv)), 0, 31). Dequantised:
    d * code + m.
    """
    x = np.asarray(x, np.float32)
    assert x.shape[-1] == BLOCK
    mn = np.min(x, axis=-1)
    mx = np.max(x, axis=-1)
    with np.errstate(over="ignore"):
        d16 = rn16((mx - mn) / np.float32(31.0))
    m16 = rn16(mn)
    zero = d16 == 0
    d_safe = np.where(zero, np.float32(1.0), d16)
    inv = np.float32(1.0) / d_safe
    diff = x - m16[..., None]                        # RN32
    prod = diff * inv[..., None]                     # RN32
    codes = np.clip(np.rint(prod), 0, 31)
    codes = np.where(zero[..., None], 0, codes).astype(np.uint8)
    d_bits = np.where(zero, np.uint16(0), f16_bits(d16)).astype(np.uint16)
    return codes, d_bits, f16_bits(m16)


def q5_1_dequantize(codes, d_bits, m_bits):
    """Dequantised Q5_1 block values d*code + m in binary64 (the product is
    exact, the sum rounds once)."""
    d = f16_from_bits(d_bits).astype(np.float64)
    m = f16_from_bits(m_bits).astype(np.float64)
    return np.asarray(codes, np.float64) * d[..., None] + m[..., None]


def q4_0_dequantize(codes, scale_bits):
    """Dequantised Q4_0 block values d*(code-8), exact in binary64."""
    d = f16_from_bits(scale_bits).astype(np.float64)
    return (np.asarray(codes, np.float64) - 8.0) * d[..., None]


# ---- page record layout (include/kvattn.h, "Pool byte layout") -------------

def _v_word_index_tables():
    """For each of the 4096 V-code words: the dim it holds and, for each of
    its 8 nibble slots j, the token slot and bit position (layout as written
    in include/kvattn.h)."""
    w = np.arange(4096)
    e = w % 4
    d = (w // 4) % 16
    g = (w // 64) % 4
    q = (w // 256) % 4
    c = w // 1024
    dim = 16 * (4 * q + e) + d
    j = np.arange(8)
    tok = 32 * c[:, None] + 16 * (j[None, :] // 4) + 4 * g[:, None] + (j[None, :] % 4)
    bit = 4 * (j // 2) + 16 * (j % 2)
    return dim, tok, bit


def _v_scale_index_tables():
    """For each of the 1024 V scales: (token slot, block) it belongs to."""
    i = np.arange(1024)
    j = i % 8
    g = (i // 8) % 4
    b = (i // 32) % 8
    c = i // 256
    tok = 32 * c + 16 * (j // 4) + 4 * g + (j % 4)
    return tok, b


_V_DIM, _V_TOK, _V_BIT = _v_word_index_tables()
_VS_TOK, _VS_BLK = _v_scale_index_tables()


def _v8_byte_index_tables():
    """For each of the 32768 code bytes of a Q8_0 value record: the token slot
    and dim it holds. Byte c*8192 + q*1024 + (16*g + r16)*16 + 8*half + j holds
    dim 32q + 16*half + r16 of slot 32c + 16*(j/4) + 4g + j%4 (include/kvattn.h)."""
    i = np.arange(V8_CODES_BYTES)
    j = i % 8
    half = (i // 8) % 2
    r16 = (i // 16) % 16
    g = (i // 256) % 4
    q = (i // 1024) % 8
    c = i // 8192
    tok = 32 * c + 16 * (j // 4) + 4 * g + (j % 4)
    dim = 32 * q + 16 * half + r16
    return tok, dim


_V8_TOK, _V8_DIM = _v8_byte_index_tables()


def pack_k_record(codes, scale_bits):
    """K record bytes from Q8_0 codes int8 [..., 128, 256] and scales uint16
    [..., 128, 8]; returns uint8 [..., 34816]."""
    codes = np.asarray(codes, np.int8)
    lead = codes.shape[:-2]
    rec = np.zeros(lead + (K_RECORD_BYTES,), np.uint8)
    rec[..., :K_CODES_BYTES] = codes.reshape(lead + (-1,)).view(np.uint8)
    sb = np.ascontiguousarray(np.asarray(scale_bits, np.uint16).astype('<u2'))
    rec[..., K_CODES_BYTES:] = sb.reshape(lead + (-1,)).view(np.uint8)
    return rec


def unpack_k_record(rec):
    """(codes int8 [..., 128, 256], scale_bits uint16 [..., 128, 8]) of K records."""
    rec = np.ascontiguousarray(np.asarray(rec, np.uint8))
    lead = rec.shape[:-1]
    codes = rec[..., :K_CODES_BYTES].view(np.int8).reshape(lead + (PAGE_TOKENS, HEAD_DIM))
    bits = np.ascontiguousarray(rec[..., K_CODES_BYTES:]).view('<u2')
    return codes.copy(), bits.reshape(lead + (PAGE_TOKENS, N_BLOCKS)).astype(np.uint16)


def pack_v_record(codes, scale_bits):
    """V record bytes from Q4_0 codes uint8 [..., 128, 256] (0..15) and scales
    uint16 [..., 128, 8]; returns uint8 [..., 18432]."""
    codes = np.asarray(codes, np.uint32)
    lead = codes.shape[:-2]
    nib = codes[..., _V_TOK, _V_DIM[:, None]]                   # [..., 4096, 8]
    words = np.zeros(lead + (4096,), np.uint32)
    for j in range(8):
        words |= nib[..., j] << np.uint32(_V_BIT[j])
    rec = np.zeros(lead + (V_RECORD_BYTES,), np.uint8)
    rec[..., :V_CODES_BYTES] = np.ascontiguousarray(words.astype('<u4')).view(np.uint8)
    sc = np.asarray(scale_bits, np.uint16)[..., _VS_TOK, _VS_BLK]
    rec[..., V_CODES_BYTES:] = np.ascontiguousarray(sc.astype('<u2')).view(np.uint8)
    return rec


def unpack_v_record(rec):
    """(codes uint8 [..., 128, 256], scale_bits uint16 [..., 128, 8]) of V records."""
    rec = np.ascontiguousarray(np.asarray(rec, np.uint8))
    lead = rec.shape[:-1]
    words = np.ascontiguousarray(rec[..., :V_CODES_BYTES]).view('<u4').astype(np.uint32)
    codes = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM), np.uint8)
    for j in range(8):
        codes[..., _V_TOK[:, j], _V_DIM] = (words >> np.uint32(_V_BIT[j])) & 0xF
    bits = np.zeros(lead + (PAGE_TOKENS, N_BLOCKS), np.uint16)
    bits[..., _VS_TOK, _VS_BLK] = np.ascontiguousarray(rec[..., V_CODES_BYTES:]).view('<u2')
    return codes, bits


def pack_v8_record(codes, scale_bits):
    """Q8_0 value record bytes from codes int8 [..., 128, 256] and scales uint16
    [..., 128, 8]; returns uint8 [..., 34816]. Scales sit after the codes in the
    Q4_0 value record's scale order."""
    codes = np.asarray(codes, np.int8)
    lead = codes.shape[:-2]
    rec = np.zeros(lead + (V8_RECORD_BYTES,), np.uint8)
    rec[..., :V8_CODES_BYTES] = np.ascontiguousarray(codes[..., _V8_TOK, _V8_DIM]).view(np.uint8)
    sc = np.asarray(scale_bits, np.uint16)[..., _VS_TOK, _VS_BLK]
    rec[..., V8_CODES_BYTES:] = np.ascontiguousarray(sc.astype('<u2')).view(np.uint8)
    return rec


def unpack_v8_record(rec):
    """(codes int8 [..., 128, 256], scale_bits uint16 [..., 128, 8]) of Q8_0 value records."""
    rec = np.ascontiguousarray(np.asarray(rec, np.uint8))
    lead = rec.shape[:-1]
    codes = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM), np.int8)
    codes[..., _V8_TOK, _V8_DIM] = rec[..., :V8_CODES_BYTES].view(np.int8)
    bits = np.zeros(lead + (PAGE_TOKENS, N_BLOCKS), np.uint16)
    bits[..., _VS_TOK, _VS_BLK] = np.ascontiguousarray(rec[..., V8_CODES_BYTES:]).view('<u2')
    return codes, bits


# Bit offset inside a 32-bit key word of dim 8w + k (k = 0..7): even k at
# 4(k/2), odd k at 16 + 4(k/2), the nibble order of the value words.
_K4_BIT = np.array([4 * (k // 2) + 16 * (k % 2) for k in range(8)], np.uint32)


def pack_k4_record(codes, scale_bits):
    """Q4_0 key record bytes from codes uint8 [..., 128, 256] (0..15) and
    scales uint16 [..., 128, 8]; returns uint8 [..., 18432]. Slot t's codes
    are the 32 little-endian words at byte t*128; word w holds dims 8w..8w+7."""
    codes = np.asarray(codes, np.uint32)
    lead = codes.shape[:-2]
    c8 = codes.reshape(lead + (PAGE_TOKENS, HEAD_DIM // 8, 8))
    words = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM // 8), np.uint32)
    for k in range(8):
        words |= (c8[..., k] & np.uint32(0xF)) << _K4_BIT[k]
    rec = np.zeros(lead + (K4_RECORD_BYTES,), np.uint8)
    rec[..., :K4_CODES_BYTES] = np.ascontiguousarray(words.astype('<u4')).reshape(
        lead + (-1,)).view(np.uint8)
    sb = np.ascontiguousarray(np.asarray(scale_bits, np.uint16).astype('<u2'))
    rec[..., K4_CODES_BYTES:] = sb.reshape(lead + (-1,)).view(np.uint8)
    return rec


def unpack_k4_record(rec):
    """(codes uint8 [..., 128, 256], scale_bits uint16 [..., 128, 8]) of Q4_0 key records."""
    rec = np.ascontiguousarray(np.asarray(rec, np.uint8))
    lead = rec.shape[:-1]
    words = np.ascontiguousarray(rec[..., :K4_CODES_BYTES]).view('<u4').astype(np.uint32)
    words = words.reshape(lead + (PAGE_TOKENS, HEAD_DIM // 8))
    codes = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM // 8, 8), np.uint8)
    for k in range(8):
        codes[..., k] = (words >> _K4_BIT[k]) & 0xF
    bits = np.ascontiguousarray(rec[..., K4_CODES_BYTES:]).view('<u2').astype(np.uint16)
    return codes.reshape(lead + (PAGE_TOKENS, HEAD_DIM)), bits.reshape(lead + (PAGE_TOKENS, N_BLOCKS))


def pack_k5_record(codes, d_bits, m_bits):
    """Q5_1 key record bytes from codes uint8 [..., 128, 256] (0..31) and
    d, m bits uint16 [..., 128, 8]; returns uint8 [..., 24576]. The low
    nibbles form a Q4_0 key record's code area; byte 16384 + t*32 + w holds
    the fifth bits of dims 8w..8w+7: dim 8w + 2p at bit p, 8w + 2p + 1 at
    bit 4 + p."""
    codes = np.asarray(codes, np.uint8)
    lead = codes.shape[:-2]
    rec = np.zeros(lead + (K5_RECORD_BYTES,), np.uint8)
    zeros = np.zeros(lead + (PAGE_TOKENS, N_BLOCKS), np.uint16)
    rec[..., :K4_CODES_BYTES] = pack_k4_record(codes & 0xF, zeros)[..., :K4_CODES_BYTES]
    hi = ((codes >> 4) & 1).reshape(lead + (PAGE_TOKENS, HEAD_DIM // 8, 8)).astype(np.uint8)
    byte = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM // 8), np.uint8)
    for k in range(8):
        byte |= hi[..., k] << np.uint8((k // 2) + 4 * (k % 2))
    rec[..., K5_HI_OFF:K5_D_OFF] = byte.reshape(lead + (-1,))
    for off, bits in ((K5_D_OFF, d_bits), (K5_M_OFF, m_bits)):
        b = np.ascontiguousarray(np.asarray(bits, np.uint16).astype('<u2'))
        rec[..., off:off + PAGE_TOKENS * N_BLOCKS * 2] = b.reshape(lead + (-1,)).view(np.uint8)
    return rec


def unpack_k5_record(rec):
    """(codes uint8 [..., 128, 256], d_bits, m_bits uint16 [..., 128, 8]) of Q5_1 key records."""
    rec = np.ascontiguousarray(np.asarray(rec, np.uint8))
    lead = rec.shape[:-1]
    k4 = np.zeros(lead + (K4_RECORD_BYTES,), np.uint8)
    k4[..., :K4_CODES_BYTES] = rec[..., :K4_CODES_BYTES]
    low, _ = unpack_k4_record(k4)
    byte = rec[..., K5_HI_OFF:K5_D_OFF].reshape(lead + (PAGE_TOKENS, HEAD_DIM // 8))
    hi = np.zeros(lead + (PAGE_TOKENS, HEAD_DIM // 8, 8), np.uint8)
    for k in range(8):
        hi[..., k] = (byte >> np.uint8((k // 2) + 4 * (k % 2))) & 1
    codes = low | (hi.reshape(lead + (PAGE_TOKENS, HEAD_DIM)) << 4)
    shp = lead + (PAGE_TOKENS, N_BLOCKS)
    d_bits = np.ascontiguousarray(rec[..., K5_D_OFF:K5_M_OFF]).view('<u2').astype(np.uint16)
    m_bits = np.ascontiguousarray(rec[..., K5_M_OFF:]).view('<u2').astype(np.uint16)
    return codes, d_bits.reshape(shp), m_bits.reshape(shp)


def key_type(k_pool):
    """'q8_0', 'q4_0' or 'q5_1' from a key pool's record size."""
    n = np.asarray(k_pool).shape[-1]
    kinds = {K_RECORD_BYTES: "q8_0", K4_RECORD_BYTES: "q4_0", K5_RECORD_BYTES: "q5_1"}
    assert n in kinds, n
    return kinds[n]


def keys_are_q4(k_pool):
    """True when a key pool (uint8 [..., record bytes]) holds Q4_0 records."""
    return key_type(k_pool) == "q4_0"


def dequantize_keys(k_records):
    """Dequantised keys (binary64) [..., 128, 256] of key records of any type."""
    kind = key_type(k_records)
    if kind == "q5_1":
        codes, db, mb = unpack_k5_record(k_records)
        lead = codes.shape[:-2]
        c = codes.reshape(lead + (PAGE_TOKENS, N_BLOCKS, BLOCK))
        return q5_1_dequantize(c, db, mb).reshape(lead + (PAGE_TOKENS, HEAD_DIM))
    codes, bits = (unpack_k4_record if kind == "q4_0" else unpack_k_record)(k_records)
    lead = codes.shape[:-2]
    dq = q4_0_dequantize if kind == "q4_0" else q8_0_dequantize
    c = codes.reshape(lead + (PAGE_TOKENS, N_BLOCKS, BLOCK))
    return dq(c, bits).reshape(lead + (PAGE_TOKENS, HEAD_DIM))


def values_are_q8(v_pool):
    """True when a value pool (uint8 [..., record bytes]) holds Q8_0 records."""
    n = np.asarray(v_pool).shape[-1]
    assert n in (V_RECORD_BYTES, V8_RECORD_BYTES), n
    return n == V8_RECORD_BYTES


def quantize_into_pool(k, v, pos0, page_table, k_pool, v_pool):
    """Write positions pos0 .. pos0+n_tok-1 into the pools (kvattn_quantize_pages
    semantics without summaries). k, v: float32 [n_tok, n_kv, 256].
    k_pool: uint8 [n_phys, n_kv, 34816] (Q8_0 keys) or [n_phys, n_kv, 18432]
    (Q4_0 keys, the value rule); v_pool: uint8 [n_phys, n_kv, 18432]
    (Q4_0 values) or [n_phys, n_kv, 34816] (Q8_0 values), both modified in
    place. Slots outside the written range keep their bytes.
    A page-table entry outside [0, n_phys) skips that page.

    [KVMEM] 測試口徑 (--kvmem-block-tokens 128: history held in 128-token
    blocks); [RDNA4] "paged decode attention". The page layout is this
    build's, written out in include/kvattn.h.
    """
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    n_tok, n_kv, D = k.shape
    assert D == HEAD_DIM and v.shape == k.shape
    n_phys = k_pool.shape[0]
    v8 = values_are_q8(v_pool)
    kind = key_type(k_pool)
    kb = k.reshape(n_tok, n_kv, N_BLOCKS, BLOCK)
    if kind == "q5_1":
        kc, ks, km = q5_1_quantize(kb)
    else:
        kc, ks = (q4_0_quantize if kind == "q4_0" else q8_0_quantize)(kb)
    vq = q8_0_quantize if v8 else q4_0_quantize
    vc, vs = vq(v.reshape(n_tok, n_kv, N_BLOCKS, BLOCK))
    kc = kc.reshape(n_tok, n_kv, HEAD_DIM)
    vc = vc.reshape(n_tok, n_kv, HEAD_DIM)
    pos = pos0 + np.arange(n_tok)
    lps = pos // PAGE_TOKENS
    pages = np.unique(lps)
    phys = np.asarray(page_table, np.int64)[pages]
    keep = (phys >= 0) & (phys < n_phys)
    pages, phys = pages[keep], phys[keep]
    if pages.size == 0:
        return
    # page index within `pages` of every token; tokens of skipped pages drop out
    where = np.searchsorted(pages, lps)
    ok = (where < pages.size) & (pages[np.minimum(where, pages.size - 1)] == lps)
    tsel = np.nonzero(ok)[0]
    pidx, slot = where[tsel], pos[tsel] % PAGE_TOKENS
    if kind == "q5_1":
        kcodes, kbits, kmins = unpack_k5_record(k_pool[phys])      # [P, n_kv, 128, ...]
    else:
        kcodes, kbits = (unpack_k4_record if kind == "q4_0" else unpack_k_record)(k_pool[phys])
    vcodes, vbits = (unpack_v8_record if v8 else unpack_v_record)(v_pool[phys])
    for h in range(n_kv):
        kcodes[pidx, h, slot] = kc[tsel, h]
        kbits[pidx, h, slot] = ks[tsel, h]
        if kind == "q5_1":
            kmins[pidx, h, slot] = km[tsel, h]
        vcodes[pidx, h, slot] = vc[tsel, h]
        vbits[pidx, h, slot] = vs[tsel, h]
    if kind == "q5_1":
        k_pool[phys] = pack_k5_record(kcodes, kbits, kmins)
    else:
        k_pool[phys] = (pack_k4_record if kind == "q4_0" else pack_k_record)(kcodes, kbits)
    v_pool[phys] = (pack_v8_record if v8 else pack_v_record)(vcodes, vbits)


def page_summaries(k_records):
    """Block summaries of full pages: RN32(binary64 sum over the 128 slots, in
    ascending slot order, of the dequantised keys, divided by 128).
    k_records uint8 [..., 34816] (Q8_0 keys) or [..., 18432] (Q4_0 keys)
    -> float32 [..., 256].

    The pages give no scoring function for KVMem ([KVMEM] "Recall 測試" only
    says retrieval picks the blocks relevant to the last user turn's query);
    the summary is the mean key of the block, the reading the workload
    description gives ("per-block summary = mean key").
    """
    lead = np.asarray(k_records).shape[:-1]
    with np.errstate(invalid="ignore", over="ignore"):   # unwritten slots: any bytes
        khat = dequantize_keys(k_records)
    acc = np.zeros(lead + (HEAD_DIM,), np.float64)
    for t in range(PAGE_TOKENS):                     # ascending t, binary64
        acc = acc + khat[..., t, :]
    return (acc / 128.0).astype(np.float32)


def page_summary(k_record):
    """Summary of one full page (page_summaries of a single record)."""
    return page_summaries(np.asarray(k_record)[None])[0]


def summaries_from_pool(k_pool, page_table, n_pages, n_kv):
    """float32 [n_kv, n_pages, 256]: summaries of logical pages 0..n_pages-1."""
    phys = np.asarray(page_table, np.int64)[:n_pages]
    return np.ascontiguousarray(np.swapaxes(page_summaries(k_pool[phys][:, :n_kv]), 0, 1))
