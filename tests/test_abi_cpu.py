"""The C-ABI library loads, exports every entry point include/kvattn.h declares,
and rejects bad arguments on the host before touching a device. No compute
call is made here (no GPU in this environment)."""
import ctypes
import os
import re

import pytest

import long_context_attention_paged_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kv.library_path()),
                                reason="libkvattn.so not built (run __graft_entry__.build())")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_DEVICE = range(5)
FAKE = 1 << 20            # a 256-byte-aligned non-null address; never dereferenced
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(kvattn_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    lib = kv.load_library()
    names = declared_functions()
    assert {"kvattn_quantize_pages", "kvattn_select_blocks", "kvattn_decode",
            "kvattn_prefill_chunk", "kvattn_merge_lse"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_count():
    lib = kv.load_library()
    for code in range(5):
        assert lib.kvattn_status_string(code)
    assert lib.kvattn_status_string(99) == b"unknown status"
    assert kv.kvattn_select_count(4088, 128, 256) == 384
    assert kv.kvattn_select_count(485, 0, 256) == 256
    assert kv.kvattn_select_count(10, 20, 5) == 10
    assert kv.kvattn_select_count(0, 1, 1) == -1
    assert kv.kvattn_select_count(5, -1, 1) == -1


def geom(n_kv=4, gqa=6, n_phys=16, head_dim=256, page=128):
    return kv.Geom(n_kv, gqa, n_phys, head_dim, page)


def decode(g, **kw):
    a = dict(q=FAKE, n_q_tok=1, k_pool=FAKE, v_pool=FAKE, table=FAKE, n_logical=16, blocks=None,
             n_blk=0, kv_len=1000, scale=0.0625, out=FAKE, lse=FAKE, n_splits=0, ws=FAKE,
             nbytes=1 << 30)
    a.update(kw)
    nb = ctypes.c_size_t(a["nbytes"])
    code = kv.load_library().kvattn_decode(
        ctypes.byref(g) if g is not None else None, P(a["q"]), a["n_q_tok"], P(a["k_pool"]),
        P(a["v_pool"]), P(a["table"]), a["n_logical"], P(a["blocks"]), a["n_blk"], a["kv_len"],
        a["scale"], P(a["out"]), P(a["lse"]), a["n_splits"], P(a["ws"]), ctypes.byref(nb), None)
    return code, nb.value


def test_decode_validation_before_device():
    assert decode(None)[0] == E_INVALID
    assert decode(geom(head_dim=128))[0] == E_UNSUPPORTED
    assert decode(geom(page=64))[0] == E_UNSUPPORTED
    assert decode(geom(n_kv=0))[0] == E_INVALID
    assert decode(geom(), n_q_tok=6)[0] == E_UNSUPPORTED       # 36 rows > 32
    assert decode(geom(gqa=33))[0] == E_UNSUPPORTED
    assert decode(geom(), n_q_tok=0)[0] == E_INVALID
    assert decode(geom(), kv_len=16 * 128 + 1)[0] == E_INVALID
    assert decode(geom(), kv_len=0)[0] == E_INVALID
    assert decode(geom(), n_q_tok=4, kv_len=3)[0] == E_INVALID
    assert decode(geom(), q=0)[0] == E_INVALID
    assert decode(geom(), q=FAKE + 4)[0] == E_INVALID          # misaligned
    assert decode(geom(), k_pool=FAKE + 16)[0] == E_INVALID    # pools need 256-byte alignment
    assert decode(geom(), blocks=FAKE, n_blk=0)[0] == E_INVALID
    assert decode(geom(), scale=float("nan"))[0] == E_INVALID
    assert decode(geom(), n_splits=-1)[0] == E_INVALID


def test_decode_workspace_protocol():
    code, need = decode(geom(), ws=None, nbytes=0, n_splits=8)
    assert code == OK
    # the 2048-byte counter area, 8 splits x 24 rows x 256 floats, plus 8 x 24 lse
    # (768 bytes, a multiple of 256)
    assert need == kv.WORKSPACE_SYNC_BYTES + 8 * 24 * 256 * 4 + 768
    code, _ = decode(geom(), n_splits=8, nbytes=need - 1)
    assert code == E_WORKSPACE
    code, need1 = decode(geom(), ws=None, nbytes=0, n_splits=0)
    assert code == OK and need1 > 0


def append_decode(g, **kw):
    a = dict(k_new=FAKE, v_new=FAKE, n_new=4, q=FAKE, n_q_tok=4, k_pool=FAKE, v_pool=FAKE,
             table=FAKE, n_logical=16, blocks=None, n_blk=0, kv_len=1000, scale=0.0625,
             summ=None, out=FAKE, lse=FAKE, n_splits=0, ws=FAKE, nbytes=1 << 30)
    a.update(kw)
    nb = ctypes.c_size_t(a["nbytes"])
    code = kv.load_library().kvattn_append_decode(
        ctypes.byref(g), P(a["k_new"]), P(a["v_new"]), a["n_new"], P(a["q"]), a["n_q_tok"],
        P(a["k_pool"]), P(a["v_pool"]), P(a["table"]), a["n_logical"], P(a["blocks"]), a["n_blk"],
        a["kv_len"], a["scale"], P(a["summ"]), P(a["out"]), P(a["lse"]), a["n_splits"],
        P(a["ws"]), ctypes.byref(nb), None)
    return code, nb.value


def test_append_decode_validation_and_workspace():
    g = geom()
    assert append_decode(g, k_new=0)[0] == E_INVALID
    assert append_decode(g, v_new=FAKE + 4)[0] == E_INVALID      # misaligned
    assert append_decode(g, n_new=0)[0] == E_INVALID
    assert append_decode(g, n_new=33)[0] == E_INVALID             # more than 32 new tokens
    assert append_decode(g, n_new=5, n_q_tok=1, kv_len=4)[0] == E_INVALID  # n_new > kv_len
    assert append_decode(g, summ=FAKE + 4)[0] == E_INVALID
    assert append_decode(g, n_q_tok=6)[0] == E_UNSUPPORTED       # decode's own checks apply
    assert append_decode(g, kv_len=16 * 128 + 1)[0] == E_INVALID
    # the workspace is kvattn_decode's
    code, need = append_decode(g, ws=None, nbytes=0, n_splits=8)
    assert code == OK and need == decode(g, ws=None, nbytes=0, n_splits=8, n_q_tok=4)[1]
    assert append_decode(g, n_splits=8, nbytes=need - 1)[0] == E_WORKSPACE


def append_decode_noalloc(g, **kw):
    a = dict(k_new=FAKE, v_new=FAKE, n_new=4, q=FAKE, n_q_tok=4, k_pool=FAKE, v_pool=FAKE,
             table=FAKE, n_logical=16, blocks=None, n_blk=0, kv_len=1000, scale=0.0625,
             summ=None, out=FAKE, lse=FAKE, n_splits=8)
    a.update(kw)
    return kv.load_library().kvattn_append_decode_noalloc(
        ctypes.byref(g), P(a["k_new"]), P(a["v_new"]), a["n_new"], P(a["q"]), a["n_q_tok"],
        P(a["k_pool"]), P(a["v_pool"]), P(a["table"]), a["n_logical"], P(a["blocks"]), a["n_blk"],
        a["kv_len"], a["scale"], P(a["summ"]), P(a["out"]), P(a["lse"]), a["n_splits"], None)


def test_append_decode_noalloc_validation():
    g = geom()
    assert append_decode_noalloc(g, k_new=0) == E_INVALID
    assert append_decode_noalloc(g, v_new=FAKE + 4) == E_INVALID
    assert append_decode_noalloc(g, n_new=0) == E_INVALID
    assert append_decode_noalloc(g, n_new=33) == E_INVALID
    assert append_decode_noalloc(g, summ=FAKE + 4) == E_INVALID
    assert append_decode_noalloc(g, out=0) == E_INVALID
    assert append_decode_noalloc(g, n_splits=-1) == E_INVALID
    assert append_decode_noalloc(g, n_q_tok=6) == E_UNSUPPORTED   # decode's own checks apply
    # partials beyond the static scratch: 64 splits x 8 KV heads x 32 rows
    # x 1028 bytes > KVATTN_NOALLOC_SCRATCH_BYTES; rejected before any device call
    g8 = geom(n_kv=8, gqa=8, n_phys=64)
    big = dict(n_q_tok=4, n_logical=64, kv_len=64 * 128, n_splits=64)
    assert append_decode_noalloc(g8, **big) == E_WORKSPACE
    assert 64 * 8 * 32 * 1028 > kv.NOALLOC_SCRATCH_BYTES >= 32 * 8 * 32 * 1028 + 512


def append_decode_partials(g, **kw):
    a = dict(k_new=FAKE, v_new=FAKE, n_new=4, q=FAKE, n_q_tok=4, k_pool=FAKE, v_pool=FAKE,
             table=FAKE, n_logical=16, blocks=None, n_blk=0, kv_len=1000, scale=0.0625,
             summ=None, n_splits=8, o_part=FAKE, lse_part=FAKE)
    a.update(kw)
    return kv.load_library().kvattn_append_decode_partials(
        ctypes.byref(g), P(a["k_new"]), P(a["v_new"]), a["n_new"], P(a["q"]), a["n_q_tok"],
        P(a["k_pool"]), P(a["v_pool"]), P(a["table"]), a["n_logical"], P(a["blocks"]), a["n_blk"],
        a["kv_len"], a["scale"], P(a["summ"]), a["n_splits"], P(a["o_part"]), P(a["lse_part"]),
        None)


def test_append_decode_partials_validation():
    g = geom()
    assert append_decode_partials(g, k_new=0) == E_INVALID
    assert append_decode_partials(g, v_new=FAKE + 4) == E_INVALID      # misaligned
    assert append_decode_partials(g, n_new=0) == E_INVALID
    assert append_decode_partials(g, n_new=33) == E_INVALID
    assert append_decode_partials(g, n_new=5, n_q_tok=1, kv_len=4) == E_INVALID
    assert append_decode_partials(g, summ=FAKE + 4) == E_INVALID
    assert append_decode_partials(g, o_part=0) == E_INVALID
    assert append_decode_partials(g, lse_part=0) == E_INVALID
    assert append_decode_partials(g, o_part=FAKE + 4) == E_INVALID    # misaligned
    assert append_decode_partials(g, n_splits=0) == E_INVALID
    assert append_decode_partials(g, n_q_tok=6) == E_UNSUPPORTED     # decode's own checks apply
    assert append_decode_partials(g, kv_len=16 * 128 + 1) == E_INVALID
    assert append_decode_partials(g, blocks=FAKE, n_blk=0) == E_INVALID


def test_prefill_range_validation():
    lib = kv.load_library()
    g = geom()

    def call(pos0=1000, chunk=100, begin=0, end=9, groups=2, n_logical=16):
        return lib.kvattn_prefill_range_partials(ctypes.byref(g), P(FAKE), chunk, P(FAKE),
                                                 P(FAKE), P(FAKE), n_logical, pos0, 0.0625,
                                                 begin, end, groups, P(FAKE), P(FAKE), None)
    # 1100 tokens -> 9 pages; the range must lie in [0, 9) and be non-empty
    assert call(end=10) == E_INVALID
    assert call(begin=-1) == E_INVALID
    assert call(begin=5, end=5) == E_INVALID
    assert call(groups=0) == E_INVALID
    assert call(pos0=2**62) == E_INVALID
    assert call() == E_DEVICE            # valid arguments reach the device check


def test_prefill_and_select_validation():
    lib = kv.load_library()
    g = geom()
    nb = ctypes.c_size_t(0)
    f = lib.kvattn_prefill_chunk
    assert f(ctypes.byref(g), P(FAKE), 0, P(FAKE), P(FAKE), P(FAKE), 16, 0, 0.0625, P(FAKE),
             P(FAKE), 0, None, ctypes.byref(nb), None) == E_INVALID           # chunk 0
    assert f(ctypes.byref(g), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16, 2000, 0.0625,
             P(FAKE), P(FAKE), 0, None, ctypes.byref(nb), None) == E_INVALID  # past the table
    assert f(ctypes.byref(g), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16, 1000, 0.0625,
             P(FAKE), P(FAKE), 4, None, ctypes.byref(nb), None) == OK
    assert nb.value == 2048 + 4 * 2400 * 256 * 4 + 4 * 2400 * 4  # counters + 4 groups x 2400 rows
    assert f(ctypes.byref(g), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16, 0, 0.0625,
             P(FAKE), P(FAKE), 4, None, ctypes.byref(nb), None) == OK
    assert nb.value == 2048 + 2400 * 256 * 4 + 9728            # groups capped at 1 page
    s = lib.kvattn_select_blocks
    assert s(ctypes.byref(g), P(FAKE), P(FAKE), 16, 17, 2, 4, P(FAKE), None, ctypes.byref(nb),
             None) == E_INVALID                                               # NB > pages
    assert s(ctypes.byref(g), P(FAKE), P(FAKE), 16, 16, -1, 4, P(FAKE), None, ctypes.byref(nb),
             None) == E_INVALID
    assert s(ctypes.byref(g), P(FAKE), P(FAKE), 16, 16, 2, 4, P(FAKE), None, ctypes.byref(nb),
             None) == OK
    assert nb.value == 2048 + 8 * 4 * 14 + (256 - (8 * 4 * 14) % 256)
    assert s(ctypes.byref(g), P(FAKE), P(FAKE), 16, 16, 2, 4, P(FAKE), P(FAKE),
             ctypes.byref(ctypes.c_size_t(8)), None) == E_WORKSPACE


def test_quantize_and_merge_validation():
    lib = kv.load_library()
    g = geom()
    q = lib.kvattn_quantize_pages
    assert q(ctypes.byref(g), P(FAKE), P(FAKE), -1, 4, P(FAKE), 16, P(FAKE), P(FAKE), None,
             None) == E_INVALID
    assert q(ctypes.byref(g), P(FAKE), P(FAKE), 2040, 9, P(FAKE), 16, P(FAKE), P(FAKE), None,
             None) == E_INVALID
    assert q(ctypes.byref(g), P(FAKE), P(FAKE), 0, 4, P(FAKE), 16, P(FAKE + 8), P(FAKE), None,
             None) == E_INVALID
    assert q(ctypes.byref(geom(head_dim=64)), P(FAKE), P(FAKE), 0, 4, P(FAKE), 16, P(FAKE),
             P(FAKE), None, None) == E_UNSUPPORTED
    m = lib.kvattn_merge_lse
    assert m(0, 4, 256, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == E_INVALID
    assert m(2, 0, 256, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == E_INVALID
    assert m(2, 4, 256, None, P(FAKE), P(FAKE), P(FAKE), None) == E_INVALID


def test_valid_call_without_device_is_a_device_error():
    """With valid arguments and no usable GPU the call reports E_DEVICE (or
    E_UNSUPPORTED on a non-gfx950 GPU) and never falls back to the CPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    lib = kv.load_library()
    code = lib.kvattn_merge_lse(2, 4, 256, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None)
    assert code in (E_DEVICE, E_UNSUPPORTED)


def test_python_binding_requires_gpu_tensors():
    import torch
    with pytest.raises((ValueError, TypeError)):
        kv.kvattn_merge_lse(torch.zeros(2, 4, 256), torch.zeros(2, 4))


def test_partials_entry_points_validate_before_device():
    import torch
    lib = kv.load_library()
    g = geom()
    d = lib.kvattn_decode_partials
    args = [ctypes.byref(g), P(FAKE), 1, P(FAKE), P(FAKE), P(FAKE), 16, None, 0, 1000, 0.0625]
    assert d(*args, 0, P(FAKE), P(FAKE), None) == E_INVALID             # n_splits 0
    assert d(*args, 4, P(FAKE + 4), P(FAKE), None) == E_INVALID         # misaligned o_part
    assert d(*args, 4, P(FAKE), None, None) == E_INVALID                # no lse_part
    assert d(ctypes.byref(geom(head_dim=128)), *args[1:], 4, P(FAKE), P(FAKE),
             None) == E_UNSUPPORTED
    p = lib.kvattn_prefill_partials
    pargs = [ctypes.byref(g), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16, 1000, 0.0625]
    assert p(*pargs, 0, P(FAKE), P(FAKE), None) == E_INVALID            # n_groups 0
    assert p(ctypes.byref(g), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16, 2000, 0.0625, 4,
             P(FAKE), P(FAKE), None) == E_INVALID                       # past the table
    if not torch.cuda.is_available():
        assert d(*args, 4, P(FAKE), P(FAKE), None) in (E_DEVICE, E_UNSUPPORTED)
        assert p(*pargs, 4, P(FAKE), P(FAKE), None) in (E_DEVICE, E_UNSUPPORTED)


def test_split_and_group_counts():
    import torch
    g = geom()
    assert kv.kvattn_decode_splits(geom(head_dim=64), 100) == 0
    assert kv.kvattn_decode_splits(g, 0) == 0
    assert kv.kvattn_decode_splits(g, 3) == 3                            # at most one per unit
    assert kv.kvattn_prefill_groups(g, 0, 0) == 0
    assert kv.kvattn_prefill_groups(g, 100, 0) == 1                      # one page
    if not torch.cuda.is_available():                                    # 256 CUs assumed
        assert kv.kvattn_decode_splits(g, 2048) == 64                    # 256 CUs / 4 heads
        # 512 x 6 rows per head in 256-row tiles: 48 tiles, about three rounds
        assert kv.kvattn_prefill_groups(g, 512, 262144) == 16


def test_prefetch_validation_before_device():
    import numpy as np
    import torch
    lib = kv.load_library()
    g = geom(n_phys=16)
    f = lib.kvattn_prefetch_pages
    pages = np.array([0, 1, 2, 15], np.int32)
    pp = pages.ctypes.data_as(ctypes.c_void_p)
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE), pp, 4, None) in \
        ((E_DEVICE, E_UNSUPPORTED) if not torch.cuda.is_available() else (OK,))
    bad = np.array([0, 16], np.int32)                                   # 16 is out of range
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
             bad.ctypes.data_as(ctypes.c_void_p), 2, None) == E_INVALID
    neg = np.array([-1], np.int32)
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
             neg.ctypes.data_as(ctypes.c_void_p), 1, None) == E_INVALID
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 3, None) == E_INVALID
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE), pp, -1, None) == E_INVALID
    assert f(ctypes.byref(g), None, P(FAKE), P(FAKE), P(FAKE), pp, 4, None) == E_INVALID
    assert f(ctypes.byref(g), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 0, None) == OK  # no-op


def test_gather_validation_before_device():
    import torch
    lib = kv.load_library()
    g = geom(n_phys=16)
    f = lib.kvattn_gather_blocks

    def call(src=FAKE, table=FAKE, n_logical=16, blocks=FAKE, n_blk=8, n_sel=4, dst=FAKE,
             dst_blocks=FAKE):
        return f(ctypes.byref(g), P(src), P(src), P(table), n_logical, P(blocks), n_blk, n_sel,
                 P(dst), P(dst), P(dst_blocks), None)

    if not torch.cuda.is_available():
        assert call() in (E_DEVICE, E_UNSUPPORTED)
    assert call(src=0) == E_INVALID
    assert call(table=0) == E_INVALID
    assert call(blocks=0) == E_INVALID
    assert call(dst_blocks=0) == E_INVALID
    assert call(n_sel=9) == E_INVALID                 # more than a row holds
    assert call(n_sel=-1) == E_INVALID
    assert call(n_blk=0, n_sel=0) == E_INVALID
    assert call(n_logical=0) == E_INVALID
    assert call(src=FAKE + 16) == E_INVALID           # pools need 256-byte alignment
    assert call(dst=FAKE + 64) == E_INVALID


def test_rotate_validation_before_device():
    import torch
    f = kv.load_library().kvattn_rotate_rows
    assert f(P(FAKE), -1, None) == E_INVALID
    assert f(None, 4, None) == E_INVALID
    assert f(P(FAKE + 4), 4, None) == E_INVALID        # misaligned
    if not torch.cuda.is_available():
        assert f(P(FAKE), 4, None) in (E_DEVICE, E_UNSUPPORTED)
        assert f(None, 0, None) in (E_DEVICE, E_UNSUPPORTED)


def test_value_type_validation():
    """v_type selects Q4_0 (0) or Q8_0 (1) value records and k_type Q8_0 (0)
    or Q4_0 (1) key records; other values are unsupported everywhere."""
    lib = kv.load_library()
    bad = geom()
    bad.v_type = 2
    assert decode(bad)[0] == E_UNSUPPORTED
    assert lib.kvattn_quantize_pages(ctypes.byref(bad), P(FAKE), P(FAKE), 0, 4, P(FAKE), 16,
                                     P(FAKE), P(FAKE), None, None) == E_UNSUPPORTED
    q8 = geom()
    q8.v_type = kv.V_Q8_0
    code, nb = decode(q8, ws=None)
    assert code == OK and nb > 0                                 # workspace query accepted
    nb = ctypes.c_size_t(0)
    assert lib.kvattn_prefill_chunk(ctypes.byref(q8), P(FAKE), 100, P(FAKE), P(FAKE), P(FAKE), 16,
                                    1000, 0.0625, P(FAKE), P(FAKE), 4, None, ctypes.byref(nb),
                                    None) == OK
    assert kv.Geom(1, 1, 1).v_record_bytes == 18432
    assert kv.Geom(1, 1, 1, v_type=kv.V_Q8_0).v_record_bytes == 34816
    assert ctypes.sizeof(kv.Geom) == 28
    badk = geom()
    q4 = geom()
    q4.k_type = kv.K_Q4_0
    code, nb = decode(q4, ws=None)
    assert code == OK and nb > 0
    assert kv.Geom(1, 1, 1, k_type=kv.K_Q4_0).k_record_bytes == 18432
    assert kv.Geom(1, 1, 1).k_record_bytes == 34816
    assert kv.Geom(1, 1, 1, k_type=kv.K_Q5_1).k_record_bytes == 24576
    q5 = geom()
    q5.k_type = kv.K_Q5_1
    assert decode(q5, ws=None)[0] == OK
    badk.k_type = 3
    assert decode(badk)[0] == E_UNSUPPORTED
