"""Shared helpers for the GPU parity tests: build matching pools on both sides
from the same seeded host inputs (the oracle quantises on the CPU, the library
on the GPU) and compare."""
import numpy as np
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv

DEV = torch.device("cuda:0")


def gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t):
    return t.detach().cpu().numpy()


class Pools:
    """A layer's pool on both sides: `ok`/`ov` are the oracle's uint8
    [n_phys, n_kv, rec] arrays, `gk`/`gv` the device copies the library writes."""

    def __init__(self, n_phys, n_kv, gqa, init_seed=None, v_type=0, k_type=0):
        self.n_phys, self.n_kv, self.gqa = n_phys, n_kv, gqa
        k_rec = {kv.K_Q4_0: quant.K4_RECORD_BYTES,
                 kv.K_Q5_1: quant.K5_RECORD_BYTES}.get(k_type, quant.K_RECORD_BYTES)
        shape_k = (n_phys, n_kv, k_rec)
        v_rec = quant.V8_RECORD_BYTES if v_type == kv.V_Q8_0 else quant.V_RECORD_BYTES
        shape_v = (n_phys, n_kv, v_rec)
        if init_seed is None:
            self.ok = np.zeros(shape_k, np.uint8)
            self.ov = np.zeros(shape_v, np.uint8)
        else:
            g = np.random.default_rng(init_seed)
            self.ok = g.integers(0, 256, shape_k, dtype=np.uint8)
            self.ov = g.integers(0, 256, shape_v, dtype=np.uint8)
        self.gk = gpu(self.ok.reshape(-1))
        self.gv = gpu(self.ov.reshape(-1))
        self.geom = kv.Geom(n_kv, gqa, n_phys, v_type=v_type, k_type=k_type)

    def write(self, K, V, pos0, table, summary=None):
        """Quantise on both sides. `summary` is a device tensor or None."""
        quant.quantize_into_pool(K, V, pos0, table, self.ok, self.ov)
        kv.kvattn_quantize_pages(self.geom, gpu(K), gpu(V), pos0, gpu(table, torch.int32),
                                 self.gk, self.gv, summary)

    def gpu_bytes(self):
        torch.cuda.synchronize()
        return (host(self.gk).reshape(self.ok.shape), host(self.gv).reshape(self.ov.shape))


def fill(n_kv, gqa, kv_len, n_phys=None, seed=0, permute=True, scale_kv=1.0, init_seed=None,
         v_type=0, k_type=0):
    """Pools holding kv_len seeded N(0,1) tokens, written in one call."""
    n_pages = (kv_len + 127) // 128
    n_phys = n_phys or n_pages + 3
    g = np.random.default_rng(seed)
    table = (g.permutation(n_phys)[:n_pages] if permute else np.arange(n_pages)).astype(np.int32)
    K = (g.standard_normal((kv_len, n_kv, 256)) * scale_kv).astype(np.float32)
    V = (g.standard_normal((kv_len, n_kv, 256)) * scale_kv).astype(np.float32)
    pools = Pools(n_phys, n_kv, gqa, init_seed, v_type, k_type)
    pools.write(K, V, 0, table)
    return pools, table, K, V


def compare(out_gpu, lse_gpu, out_ref, lse_ref):
    """(max-abs out error, max-abs lse error, relative RMS out error)."""
    o, l_ = host(out_gpu).astype(np.float64), host(lse_gpu).astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(l_) == np.isneginf(lse_ref)).all(), "empty rows disagree"
    eo = np.abs(o - out_ref).max()
    el = np.abs(l_[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    rr = np.sqrt(((o - out_ref) ** 2).sum() / max((out_ref ** 2).sum(), 1e-300))
    return eo, el, rr


def prefill_checked(geom, q, k_pool, v_pool, page_table, pos0, scale, n_groups=0):
    """kvattn_prefill_chunk on a fresh zeroed workspace; asserts afterwards that
    no wavefront's bounded wait gave up (the workspace's error word is 0)."""
    import ctypes
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    nb = ctypes.c_size_t(0)
    code = kv.load_library().kvattn_prefill_chunk(
        ctypes.byref(geom), ctypes.c_void_p(q.data_ptr()), q.shape[0],
        ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
        ctypes.c_void_p(page_table.data_ptr()), page_table.numel(), int(pos0), float(scale),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()), int(n_groups), None,
        ctypes.byref(nb), None)
    assert code == 0, code
    ws = kv.workspace(nb.value, q.device)
    out, lse = kv.kvattn_prefill_chunk(geom, q, k_pool, v_pool, page_table, pos0, scale,
                                       out=out, lse=lse, n_groups=n_groups, workspace=ws)
    assert kv.workspace_error(ws) == 0, "a prefill wavefront's wait gave up"
    return out, lse
