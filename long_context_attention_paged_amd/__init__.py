"""Paged Q8_0/Q4_0 attention for MI355X (gfx950): thin Python binding of
libkvattn.so (include/kvattn.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. Tensors are torch tensors on the current GPU; outputs and workspaces
that are not passed in are allocated with torch (device memory plumbing) and
work is enqueued on torch's current stream. If the library is not built, or
the device is not gfx950, calls raise: there is no CPU fallback.
"""
import ctypes
import os

__all__ = [
    "Geom", "KvattnError", "library_path", "load_library",
    "kvattn_quantize_pages", "kvattn_select_blocks", "kvattn_decode",
    "kvattn_decode_partials", "kvattn_append_decode_partials", "kvattn_decode_splits",
    "kvattn_prefill_chunk",
    "kvattn_prefill_partials", "kvattn_prefill_groups", "kvattn_merge_lse",
    "kvattn_prefetch_pages", "kvattn_select_count", "workspace", "workspace_error",
    "K_RECORD_BYTES", "V_RECORD_BYTES", "HEAD_DIM", "PAGE_TOKENS",
]

HEAD_DIM = 256
PAGE_TOKENS = 128
K_RECORD_BYTES = 34816
V_RECORD_BYTES = 18432
V8_RECORD_BYTES = 34816
V_Q4_0, V_Q8_0 = 0, 1  # value cache types (kvattn_geom.v_type)
K4_RECORD_BYTES = 18432
K5_RECORD_BYTES = 24576
K_Q8_0, K_Q4_0, K_Q5_1 = 0, 1, 2  # key cache types (kvattn_geom.k_type)
STATUS = {0: "OK", 1: "E_INVALID", 2: "E_UNSUPPORTED", 3: "E_WORKSPACE", 4: "E_DEVICE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class KvattnError(RuntimeError):
    def __init__(self, func, code):
        self.code = code
        super().__init__(f"{func} failed: {STATUS.get(code, code)}")


class Geom(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("gqa", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("n_phys_pages", ctypes.c_int32), ("v_type", ctypes.c_int32),
                ("k_type", ctypes.c_int32)]

    def __init__(self, n_kv_heads, gqa, n_phys_pages, head_dim=HEAD_DIM, page_tokens=PAGE_TOKENS,
                 v_type=0, k_type=0):
        super().__init__(n_kv_heads, gqa, head_dim, page_tokens, n_phys_pages, v_type, k_type)

    @property
    def k_record_bytes(self):
        return {K_Q4_0: K4_RECORD_BYTES, K_Q5_1: K5_RECORD_BYTES}.get(self.k_type, K_RECORD_BYTES)

    @property
    def v_record_bytes(self):
        return V8_RECORD_BYTES if self.v_type == V_Q8_0 else V_RECORD_BYTES


def library_path():
    return os.path.join(_HERE, "libkvattn.so")


def load_library():
    """Load libkvattn.so (built by build.py) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run long_context_attention_paged_amd/build.py")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZP = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.POINTER(ctypes.c_size_t))
    G = ctypes.POINTER(Geom)
    sigs = {
        "kvattn_status_string": ([I32], ctypes.c_char_p),
        "kvattn_select_count": ([I32, I32, I32], I32),
        "kvattn_quantize_pages": ([G, P, P, I64, I32, P, I32, P, P, P, P], I32),
        "kvattn_select_blocks": ([G, P, P, I32, I32, I32, I32, P, P, SZP, P], I32),
        "kvattn_decode": ([G, P, I32, P, P, P, I32, P, I32, I64, F32, P, P, I32, P, SZP, P], I32),
        "kvattn_decode_partials": ([G, P, I32, P, P, P, I32, P, I32, I64, F32, I32, P, P, P], I32),
        "kvattn_append_decode": ([G, P, P, I32, P, I32, P, P, P, I32, P, I32, I64, F32, P, P, P,
                                  I32, P, SZP, P], I32),
        "kvattn_append_decode_noalloc": ([G, P, P, I32, P, I32, P, P, P, I32, P, I32, I64, F32, P,
                                          P, P, I32, P], I32),
        "kvattn_append_decode_partials": ([G, P, P, I32, P, I32, P, P, P, I32, P, I32, I64, F32,
                                           P, I32, P, P, P], I32),
        "kvattn_decode_splits": ([G, I32], I32),
        "kvattn_prefill_chunk": ([G, P, I32, P, P, P, I32, I64, F32, P, P, I32, P, SZP, P], I32),
        "kvattn_prefill_partials": ([G, P, I32, P, P, P, I32, I64, F32, I32, P, P, P], I32),
        "kvattn_prefill_range_partials": ([G, P, I32, P, P, P, I32, I64, F32, I32, I32, I32, P,
                                           P, P], I32),
        "kvattn_prefill_groups": ([G, I32, I64], I32),
        "kvattn_merge_lse": ([I32, I64, I32, P, P, P, P, P], I32),
        "kvattn_prefetch_pages": ([G, P, P, P, P, P, I32, P], I32),
        "kvattn_gather_blocks": ([G, P, P, P, I32, P, I32, I32, P, P, P, P], I32),
        "kvattn_rotate_rows": ([P, I64, P], I32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


# ---- marshalling helpers ---------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _size(t, name, need):
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {need}")


def _pools(geom, k_pool, v_pool):
    _size(k_pool, "k_pool", geom.n_phys_pages * geom.n_kv_heads * geom.k_record_bytes)
    _size(v_pool, "v_pool", geom.n_phys_pages * geom.n_kv_heads * geom.v_record_bytes)


def _check(func, code):
    if code != 0:
        raise KvattnError(func, code)


WORKSPACE_SYNC_BYTES = 2048  # counters at the start of every workspace (include/kvattn.h)
NOALLOC_SCRATCH_BYTES = 16 << 20  # the static partials of kvattn_append_decode_noalloc


def workspace(nbytes, device):
    """A workspace of nbytes (at least the counter area), zeroed as the
    library requires before its first use."""
    torch = _torch()
    return torch.zeros(max(int(nbytes), WORKSPACE_SYNC_BYTES), dtype=torch.uint8, device=device)


def workspace_error(ws):
    """The workspace's error word (bytes 0..3): bit 0 is set by a prefill
    launch whose bounded waits gave up (never expected). Synchronises with
    the device."""
    return int(ws[:4].view(_torch().int32).item())


def _workspace(query, ws, device):
    """Size the workspace with a NULL query, allocate it (zeroed) if not given."""
    torch = _torch()
    size = ctypes.c_size_t(0)
    _check("workspace query", query(None, ctypes.byref(size)))
    if ws is None:
        ws = workspace(int(size.value), device)
    _need(ws, "workspace", torch.uint8)
    return ws, ctypes.c_size_t(ws.numel())


def kvattn_select_count(n_blocks, n_recent, k_top):
    return int(load_library().kvattn_select_count(n_blocks, n_recent, k_top))


def kvattn_quantize_pages(geom, k, v, pos0, page_table, k_pool, v_pool, k_summary=None,
                          stream=None):
    """Quantise positions pos0 .. pos0+k.shape[0]-1 into the pools (a1)."""
    torch = _torch()
    lib = load_library()
    for name, t, dt in (("k", k, torch.float32), ("v", v, torch.float32),
                        ("page_table", page_table, torch.int32),
                        ("k_pool", k_pool, torch.uint8), ("v_pool", v_pool, torch.uint8)):
        _need(t, name, dt)
    n_tok = k.shape[0]
    _size(k, "k", n_tok * geom.n_kv_heads * HEAD_DIM)
    _size(v, "v", n_tok * geom.n_kv_heads * HEAD_DIM)
    _pools(geom, k_pool, v_pool)
    if k_summary is not None:
        _need(k_summary, "k_summary", torch.float32)
        _size(k_summary, "k_summary", geom.n_kv_heads * page_table.numel() * HEAD_DIM)
    code = lib.kvattn_quantize_pages(ctypes.byref(geom), _ptr(k), _ptr(v), int(pos0), k.shape[0],
                                     _ptr(page_table), page_table.numel(), _ptr(k_pool),
                                     _ptr(v_pool), _ptr(k_summary), _stream(stream))
    _check("kvattn_quantize_pages", code)


def kvattn_select_blocks(geom, q, k_summary, n_logical_pages, n_blocks, n_recent, k_top,
                         out_blocks=None, workspace=None, stream=None):
    """KVMem block selection (a2); returns int32 [n_kv, count] ascending blocks."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.float32)
    _need(k_summary, "k_summary", torch.float32)
    n_out = kvattn_select_count(n_blocks, n_recent, k_top)
    if n_out < 0:
        raise ValueError("invalid selection sizes")
    _size(q, "q", geom.n_kv_heads * geom.gqa * HEAD_DIM)
    _size(k_summary, "k_summary", geom.n_kv_heads * n_logical_pages * HEAD_DIM)
    if out_blocks is None:
        out_blocks = torch.empty((geom.n_kv_heads, max(n_out, 1)), dtype=torch.int32,
                                 device=q.device)
    _need(out_blocks, "out_blocks", torch.int32)
    if out_blocks.dim() != 2 or out_blocks.shape[0] != geom.n_kv_heads or \
            out_blocks.shape[1] < n_out:
        raise ValueError("out_blocks must be [n_kv_heads, >= count]")
    if out_blocks.shape[1] != max(n_out, 1):
        raise ValueError("out_blocks rows must hold exactly kvattn_select_count() entries")
    if n_out == 0:
        return out_blocks[:, :0]

    def call(ws, nbytes):
        return lib.kvattn_select_blocks(ctypes.byref(geom), _ptr(q), _ptr(k_summary),
                                        n_logical_pages, n_blocks, n_recent, k_top,
                                        _ptr(out_blocks), ws, nbytes, _stream(stream))

    workspace, nbytes = _workspace(call, workspace, q.device)
    _check("kvattn_select_blocks", call(_ptr(workspace), ctypes.byref(nbytes)))
    return out_blocks[:, :n_out]


def kvattn_decode(geom, q, k_pool, v_pool, page_table, kv_len, scale, blocks=None, out=None,
                  lse=None, n_splits=0, workspace=None, stream=None):
    """Decode / verify attention (a3, a5); q [n_q_tok, n_heads, 256] -> (out, lse)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.float32)
    for name, t, dt in (("k_pool", k_pool, torch.uint8), ("v_pool", v_pool, torch.uint8),
                        ("page_table", page_table, torch.int32)):
        _need(t, name, dt)
    n_q_tok = q.shape[0]
    n_heads = geom.n_kv_heads * geom.gqa
    if q.dim() != 3 or q.shape[1] != n_heads or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [n_q_tok, {n_heads}, {HEAD_DIM}]")
    _pools(geom, k_pool, v_pool)
    n_blk = 0
    if blocks is not None:
        _need(blocks, "blocks", torch.int32)
        if blocks.dim() != 2 or blocks.shape[0] != geom.n_kv_heads:
            raise ValueError("blocks must be [n_kv_heads, n_blk]")
        n_blk = blocks.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _size(out, "out", q.numel())
    _size(lse, "lse", n_q_tok * n_heads)

    def call(ws, nbytes):
        return lib.kvattn_decode(ctypes.byref(geom), _ptr(q), n_q_tok, _ptr(k_pool), _ptr(v_pool),
                                 _ptr(page_table), page_table.numel(), _ptr(blocks), n_blk,
                                 int(kv_len), float(scale), _ptr(out), _ptr(lse), int(n_splits),
                                 ws, nbytes, _stream(stream))

    workspace, nbytes = _workspace(call, workspace, q.device)
    _check("kvattn_decode", call(_ptr(workspace), ctypes.byref(nbytes)))
    return out, lse


def kvattn_append_decode(geom, k_new, v_new, q, k_pool, v_pool, page_table, kv_len, scale,
                         blocks=None, k_summary=None, out=None, lse=None, n_splits=0,
                         workspace=None, stream=None):
    """Append then decode in one launch (a1 + a3/a5): k_new, v_new [n_new, n_kv, 256]
    are the keys and values of positions kv_len - n_new .. kv_len - 1; -> (out, lse)."""
    torch = _torch()
    lib = load_library()
    n_blk = _decode_args(geom, q, k_pool, v_pool, page_table, blocks)
    n_new = k_new.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, torch.float32)
        _size(t, name, n_new * geom.n_kv_heads * HEAD_DIM)
    if k_summary is not None:
        _need(k_summary, "k_summary", torch.float32)
        _size(k_summary, "k_summary", geom.n_kv_heads * page_table.numel() * HEAD_DIM)
    n_q_tok = q.shape[0]
    n_heads = geom.n_kv_heads * geom.gqa
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _size(out, "out", q.numel())
    _size(lse, "lse", n_q_tok * n_heads)

    def call(ws, nbytes):
        return lib.kvattn_append_decode(ctypes.byref(geom), _ptr(k_new), _ptr(v_new), n_new,
                                        _ptr(q), n_q_tok, _ptr(k_pool), _ptr(v_pool),
                                        _ptr(page_table), page_table.numel(), _ptr(blocks), n_blk,
                                        int(kv_len), float(scale), _ptr(k_summary), _ptr(out),
                                        _ptr(lse), int(n_splits), ws, nbytes, _stream(stream))

    workspace, nbytes = _workspace(call, workspace, q.device)
    _check("kvattn_append_decode", call(_ptr(workspace), ctypes.byref(nbytes)))
    return out, lse


def kvattn_append_decode_noalloc(geom, k_new, v_new, q, k_pool, v_pool, page_table, kv_len,
                                 scale, out, lse, blocks=None, k_summary=None, n_splits=0,
                                 stream=None):
    """kvattn_append_decode with its partials in the library's static
    per-GPU scratch: no workspace, and no allocation here either, so out and
    lse are required. Raises KvattnError (KVATTN_E_WORKSPACE) when the
    partials exceed NOALLOC_SCRATCH_BYTES."""
    torch = _torch()
    lib = load_library()
    n_blk = _decode_args(geom, q, k_pool, v_pool, page_table, blocks)
    n_new = k_new.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, torch.float32)
        _size(t, name, n_new * geom.n_kv_heads * HEAD_DIM)
    if k_summary is not None:
        _need(k_summary, "k_summary", torch.float32)
        _size(k_summary, "k_summary", geom.n_kv_heads * page_table.numel() * HEAD_DIM)
    n_q_tok = q.shape[0]
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _size(out, "out", q.numel())
    _size(lse, "lse", n_q_tok * geom.n_kv_heads * geom.gqa)
    _check("kvattn_append_decode_noalloc",
           lib.kvattn_append_decode_noalloc(ctypes.byref(geom), _ptr(k_new), _ptr(v_new), n_new,
                                            _ptr(q), n_q_tok, _ptr(k_pool), _ptr(v_pool),
                                            _ptr(page_table), page_table.numel(), _ptr(blocks),
                                            n_blk, int(kv_len), float(scale), _ptr(k_summary),
                                            _ptr(out), _ptr(lse), int(n_splits),
                                            _stream(stream)))
    return out, lse


def _decode_args(geom, q, k_pool, v_pool, page_table, blocks):
    torch = _torch()
    _need(q, "q", torch.float32)
    for name, t, dt in (("k_pool", k_pool, torch.uint8), ("v_pool", v_pool, torch.uint8),
                        ("page_table", page_table, torch.int32)):
        _need(t, name, dt)
    n_heads = geom.n_kv_heads * geom.gqa
    if q.dim() != 3 or q.shape[1] != n_heads or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [n_q_tok, {n_heads}, {HEAD_DIM}]")
    _pools(geom, k_pool, v_pool)
    n_blk = 0
    if blocks is not None:
        _need(blocks, "blocks", torch.int32)
        if blocks.dim() != 2 or blocks.shape[0] != geom.n_kv_heads:
            raise ValueError("blocks must be [n_kv_heads, n_blk]")
        n_blk = blocks.shape[1]
    return n_blk


def kvattn_append_decode_partials(geom, k_new, v_new, q, k_pool, v_pool, page_table, kv_len,
                                  scale, n_splits, blocks=None, k_summary=None, o_part=None,
                                  lse_part=None, stream=None):
    """The append of kvattn_append_decode with the partials of kvattn_decode_partials
    (a1 + a3), no merge: -> (o_part [n_splits, n_q_tok*n_heads, 256], lse_part)."""
    torch = _torch()
    lib = load_library()
    n_blk = _decode_args(geom, q, k_pool, v_pool, page_table, blocks)
    n_new = k_new.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, torch.float32)
        _size(t, name, n_new * geom.n_kv_heads * HEAD_DIM)
    if k_summary is not None:
        _need(k_summary, "k_summary", torch.float32)
        _size(k_summary, "k_summary", geom.n_kv_heads * page_table.numel() * HEAD_DIM)
    rows = q.shape[0] * q.shape[1]
    if o_part is None:
        o_part = torch.empty((n_splits, rows, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n_splits, rows), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _size(o_part, "o_part", n_splits * rows * HEAD_DIM)
    _size(lse_part, "lse_part", n_splits * rows)
    _check("kvattn_append_decode_partials",
           lib.kvattn_append_decode_partials(
               ctypes.byref(geom), _ptr(k_new), _ptr(v_new), n_new, _ptr(q), q.shape[0],
               _ptr(k_pool), _ptr(v_pool), _ptr(page_table), page_table.numel(), _ptr(blocks),
               n_blk, int(kv_len), float(scale), _ptr(k_summary), int(n_splits), _ptr(o_part),
               _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def kvattn_decode_splits(geom, n_units):
    """Split count kvattn_decode picks by itself for n_units pages or blocks."""
    return load_library().kvattn_decode_splits(ctypes.byref(geom), int(n_units))


def kvattn_decode_partials(geom, q, k_pool, v_pool, page_table, kv_len, scale, n_splits,
                           blocks=None, o_part=None, lse_part=None, stream=None):
    """Split-K partials of decode (a3) without the merge:
    q [n_q_tok, n_heads, 256] -> (o_part [n_splits, n_q_tok*n_heads, 256], lse_part)."""
    torch = _torch()
    lib = load_library()
    n_blk = _decode_args(geom, q, k_pool, v_pool, page_table, blocks)
    rows = q.shape[0] * q.shape[1]
    if o_part is None:
        o_part = torch.empty((n_splits, rows, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n_splits, rows), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _size(o_part, "o_part", n_splits * rows * HEAD_DIM)
    _size(lse_part, "lse_part", n_splits * rows)
    _check("kvattn_decode_partials",
           lib.kvattn_decode_partials(ctypes.byref(geom), _ptr(q), q.shape[0], _ptr(k_pool),
                                      _ptr(v_pool), _ptr(page_table), page_table.numel(),
                                      _ptr(blocks), n_blk, int(kv_len), float(scale),
                                      int(n_splits), _ptr(o_part), _ptr(lse_part),
                                      _stream(stream)))
    return o_part, lse_part


def kvattn_prefill_chunk(geom, q, k_pool, v_pool, page_table, pos0, scale, out=None, lse=None,
                         n_groups=0, workspace=None, stream=None):
    """Chunked prefill attention (a6); q [chunk, n_heads, 256] -> (out, lse)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.float32)
    for name, t, dt in (("k_pool", k_pool, torch.uint8), ("v_pool", v_pool, torch.uint8),
                        ("page_table", page_table, torch.int32)):
        _need(t, name, dt)
    n_heads = geom.n_kv_heads * geom.gqa
    if q.dim() != 3 or q.shape[1] != n_heads or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [chunk, {n_heads}, {HEAD_DIM}]")
    _pools(geom, k_pool, v_pool)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _size(out, "out", q.numel())
    _size(lse, "lse", q.shape[0] * n_heads)

    def call(ws, nbytes):
        return lib.kvattn_prefill_chunk(ctypes.byref(geom), _ptr(q), q.shape[0], _ptr(k_pool),
                                        _ptr(v_pool), _ptr(page_table), page_table.numel(),
                                        int(pos0), float(scale), _ptr(out), _ptr(lse),
                                        int(n_groups), ws, nbytes, _stream(stream))

    workspace, nbytes = _workspace(call, workspace, q.device)
    _check("kvattn_prefill_chunk", call(_ptr(workspace), ctypes.byref(nbytes)))
    return out, lse


def prefill_workspace_bytes(geom, q, k_pool, v_pool, page_table, pos0, n_groups=0):
    """Workspace bytes kvattn_prefill_chunk needs for these arguments (its
    NULL-workspace query; nothing is enqueued)."""
    lib = load_library()
    n_heads = geom.n_kv_heads * geom.gqa
    size = ctypes.c_size_t(0)
    # out and lse are only checked for presence by the query
    _check("kvattn_prefill_chunk", lib.kvattn_prefill_chunk(
        ctypes.byref(geom), _ptr(q), q.shape[0], _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
        page_table.numel(), int(pos0), 1.0, _ptr(q), _ptr(q), int(n_groups), None,
        ctypes.byref(size), None))
    assert q.shape[1] == n_heads
    return int(size.value)


def kvattn_prefill_groups(geom, chunk, pos0):
    """Page-group count kvattn_prefill_chunk picks by itself."""
    return load_library().kvattn_prefill_groups(ctypes.byref(geom), int(chunk), int(pos0))


def kvattn_prefill_partials(geom, q, k_pool, v_pool, page_table, pos0, scale, n_groups,
                            o_part=None, lse_part=None, stream=None):
    """Per-group partials of chunked prefill (a6) without the merge:
    q [chunk, n_heads, 256] -> (o_part [n_groups, chunk*n_heads, 256], lse_part)."""
    torch = _torch()
    lib = load_library()
    _decode_args(geom, q, k_pool, v_pool, page_table, None)
    rows = q.shape[0] * q.shape[1]
    if o_part is None:
        o_part = torch.empty((n_groups, rows, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n_groups, rows), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _size(o_part, "o_part", n_groups * rows * HEAD_DIM)
    _size(lse_part, "lse_part", n_groups * rows)
    _check("kvattn_prefill_partials",
           lib.kvattn_prefill_partials(ctypes.byref(geom), _ptr(q), q.shape[0], _ptr(k_pool),
                                       _ptr(v_pool), _ptr(page_table), page_table.numel(),
                                       int(pos0), float(scale), int(n_groups), _ptr(o_part),
                                       _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def kvattn_prefill_range_partials(geom, q, k_pool, v_pool, page_table, pos0, scale, page_begin,
                                  page_end, n_groups, o_part=None, lse_part=None, stream=None):
    """Prefill partials over the keys of logical pages [page_begin, page_end)
    only (a6 over a page range): -> (o_part [n_groups, chunk*n_heads, 256],
    lse_part); the pool and table need to hold only that range's pages."""
    torch = _torch()
    lib = load_library()
    _decode_args(geom, q, k_pool, v_pool, page_table, None)
    rows = q.shape[0] * q.shape[1]
    if o_part is None:
        o_part = torch.empty((n_groups, rows, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n_groups, rows), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _size(o_part, "o_part", n_groups * rows * HEAD_DIM)
    _size(lse_part, "lse_part", n_groups * rows)
    _check("kvattn_prefill_range_partials",
           lib.kvattn_prefill_range_partials(ctypes.byref(geom), _ptr(q), q.shape[0], _ptr(k_pool),
                                             _ptr(v_pool), _ptr(page_table), page_table.numel(),
                                             int(pos0), float(scale), int(page_begin),
                                             int(page_end), int(n_groups), _ptr(o_part),
                                             _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def kvattn_merge_lse(o_parts, lse_parts, out=None, lse=None, stream=None):
    """LSE merge (a4): o_parts [S, rows, D], lse_parts [S, rows] -> (out, lse)."""
    torch = _torch()
    lib = load_library()
    _need(o_parts, "o_parts", torch.float32)
    _need(lse_parts, "lse_parts", torch.float32)
    S, rows, D = o_parts.shape
    if out is None:
        out = torch.empty((rows, D), dtype=torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _size(out, "out", rows * D)
    _size(lse, "lse", rows)
    _size(lse_parts, "lse_parts", S * rows)
    code = lib.kvattn_merge_lse(S, rows, D, _ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse),
                                _stream(stream))
    _check("kvattn_merge_lse", code)
    return out, lse


def kvattn_rotate_rows(x, stream=None):
    """In-place Hadamard rotation H_256 / 16 of every 256-element row of the
    fp32 device tensor x (keys before quantisation, queries before attention)."""
    torch = _torch()
    lib = load_library()
    _need(x, "x", torch.float32)
    if x.numel() % HEAD_DIM:
        raise ValueError(f"x must hold whole rows of {HEAD_DIM} elements")
    _check("kvattn_rotate_rows",
           lib.kvattn_rotate_rows(_ptr(x), x.numel() // HEAD_DIM, _stream(stream)))
    return x


def kvattn_gather_blocks(geom, src_k_pool, src_v_pool, page_table, blocks, n_sel, dst_k_pool,
                         dst_v_pool, dst_blocks=None, stream=None):
    """KVMem host tier: copy the first n_sel blocks of each head's row of
    `blocks` (device [n_kv, n_blk]) from the src pools (device, or pinned host
    tensors) into ranks 0..n_sel-1 of the dst pools -> dst_blocks [n_kv, n_sel]."""
    torch = _torch()
    lib = load_library()
    for name, t in (("src_k_pool", src_k_pool), ("src_v_pool", src_v_pool)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous uint8 torch tensor")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    _pools(geom, src_k_pool, src_v_pool)
    _need(page_table, "page_table", torch.int32)
    _need(blocks, "blocks", torch.int32)
    if blocks.dim() != 2 or blocks.shape[0] != geom.n_kv_heads:
        raise ValueError("blocks must be [n_kv_heads, n_blk]")
    n_sel = int(n_sel)
    _need(dst_k_pool, "dst_k_pool", torch.uint8)
    _need(dst_v_pool, "dst_v_pool", torch.uint8)
    _size(dst_k_pool, "dst_k_pool", n_sel * geom.n_kv_heads * geom.k_record_bytes)
    _size(dst_v_pool, "dst_v_pool", n_sel * geom.n_kv_heads * geom.v_record_bytes)
    if dst_blocks is None:
        dst_blocks = torch.empty((geom.n_kv_heads, max(n_sel, 1)), dtype=torch.int32,
                                 device=blocks.device)
    _need(dst_blocks, "dst_blocks", torch.int32)
    _size(dst_blocks, "dst_blocks", geom.n_kv_heads * n_sel)
    _check("kvattn_gather_blocks",
           lib.kvattn_gather_blocks(ctypes.byref(geom), _ptr(src_k_pool), _ptr(src_v_pool),
                                    _ptr(page_table), page_table.numel(), _ptr(blocks),
                                    blocks.shape[1], n_sel, _ptr(dst_k_pool), _ptr(dst_v_pool),
                                    _ptr(dst_blocks), _stream(stream)))
    return dst_blocks


def kvattn_prefetch_pages(geom, src_k_pool, src_v_pool, dst_k_pool, dst_v_pool, pages,
                          stream=None):
    """Page prefetch (a7): copy the records of physical `pages` (a host
    sequence of ints) from the src pools to the dst pools, asynchronously on
    `stream`. Each pool is a device tensor or a pinned host tensor: typically
    host to device, and device to host to write pages back."""
    import numpy as np
    torch = _torch()
    lib = load_library()
    for name, t in (("src_k_pool", src_k_pool), ("src_v_pool", src_v_pool),
                    ("dst_k_pool", dst_k_pool), ("dst_v_pool", dst_v_pool)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous uint8 torch tensor")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    _pools(geom, dst_k_pool, dst_v_pool)
    _pools(geom, src_k_pool, src_v_pool)
    idx = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
    _check("kvattn_prefetch_pages",
           lib.kvattn_prefetch_pages(ctypes.byref(geom), _ptr(src_k_pool), _ptr(src_v_pool),
                                     _ptr(dst_k_pool), _ptr(dst_v_pool),
                                     idx.ctypes.data_as(ctypes.c_void_p), int(idx.size),
                                     _stream(stream)))
