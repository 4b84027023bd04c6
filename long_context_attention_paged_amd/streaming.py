"""Adaptive host-resident KV streaming for decode and verify steps.

The Adaptive KV Streaming pages ([STREAM] "先說結論"; [RDNA4] the design
bullets) keep the full KV history in pinned host memory and hold only a
bounded working set on the GPU, streamed over PCIe alongside compute. This
module composes the library's entry points into that regime for one
sequence; every byte of attention still runs in the library's kernels and
every copy is the library's hipMemcpyAsync:

 - per layer, the newest `n_res` pages stay resident in a compact device
   pool (its page table maps the resident logical pages to slots, every other
   page to -1); the appended tokens land there;
 - the older `n_hist` pages live in a pinned host tier in logical order, so
   one layer's history is one contiguous copy per pool;
 - per step and layer, a copy stream moves the layer's history into one of
   two device staging pools (layer L+1 copies while layer L computes), and
   the compute stream runs kvattn_append_decode over the resident pages and
   kvattn_decode_partials over the staged history, then kvattn_merge_lse of
   the two, which is exact (the LSE merge is associative over any page split).

Device working set: n_layers * n_res pages resident plus 2 * n_hist staged.
"""
import numpy as np

import long_context_attention_paged_amd as kv

K_REC, V_REC = kv.K_RECORD_BYTES, kv.V_RECORD_BYTES
PAGE = kv.PAGE_TOKENS


def resident_pages_for_budget(budget_bytes, n_layers, n_pages, n_kv, v_record_bytes=V_REC,
                              k_record_bytes=K_REC):
    """Largest n_res such that n_layers * n_res resident pages plus two staging
    pools of n_pages - n_res pages fit in budget_bytes (at least one page)."""
    page = n_kv * (k_record_bytes + v_record_bytes)
    n_res = (budget_bytes // page - 2 * n_pages) // (n_layers - 2) if n_layers > 2 else n_pages
    return int(max(1, min(n_pages, n_res)))


class StreamedLayer:
    """One layer's two tiers, built from a full device pool (k_pool, v_pool,
    page_table over n_pages logical pages): history pages [0, n_hist) go to
    pinned host memory in logical order (unless keep_history is False), pages
    [n_hist, n_pages) to a compact device pool."""

    def __init__(self, geom, k_pool, v_pool, page_table, n_pages, n_hist, keep_history=True):
        import torch
        dev = k_pool.device
        n_kv = geom.n_kv_heads
        table = torch.as_tensor(page_table, device=dev).long()
        kview = k_pool.view(-1, n_kv * geom.k_record_bytes)
        vview = v_pool.view(-1, n_kv * geom.v_record_bytes)
        hist, res = table[:n_hist], table[n_hist:n_pages]
        self.n_hist, self.n_res = n_hist, n_pages - n_hist
        self.host_k = self.host_v = None
        if keep_history:
            self.host_k = torch.empty(max(n_hist, 1) * n_kv * geom.k_record_bytes,
                                      dtype=torch.uint8, pin_memory=True)
            self.host_v = torch.empty(max(n_hist, 1) * n_kv * geom.v_record_bytes,
                                      dtype=torch.uint8, pin_memory=True)
        if n_hist and keep_history:
            self.host_k[:n_hist * n_kv * geom.k_record_bytes].copy_(kview[hist].reshape(-1))
            self.host_v[:n_hist * n_kv * geom.v_record_bytes].copy_(vview[hist].reshape(-1))
        self.res_k = kview[res].reshape(-1).contiguous()
        self.res_v = vview[res].reshape(-1).contiguous()
        rt = np.full(n_pages, -1, np.int32)
        rt[n_hist:] = np.arange(self.n_res, dtype=np.int32)
        self.res_table = torch.from_numpy(rt).to(dev)
        self.res_blocks = torch.from_numpy(
            np.tile(np.arange(n_hist, n_pages, dtype=np.int32), (n_kv, 1))).to(dev)
        self.res_geom = kv.Geom(n_kv, geom.gqa, self.n_res, v_type=geom.v_type,
                                k_type=geom.k_type)
        torch.cuda.synchronize()


class StreamedDecode:
    """Decode / verify over streamed layers. `layers` are StreamedLayer objects
    with the same n_hist; q, k_new, v_new, out and lse are per-layer lists."""

    def __init__(self, geom, layers, n_pages, n_q_tok, dev, workspace_bytes=64 << 20):
        import torch
        self.layers = layers
        self.n_hist = layers[0].n_hist
        self.n_pages = n_pages
        n_kv = geom.n_kv_heads
        self.hist_geom = kv.Geom(n_kv, geom.gqa, max(self.n_hist, 1), v_type=geom.v_type,
                                 k_type=geom.k_type)
        self.stage_k = [torch.empty(max(self.n_hist, 1) * n_kv * geom.k_record_bytes,
                                    dtype=torch.uint8, device=dev) for _ in range(2)]
        self.stage_v = [torch.empty(max(self.n_hist, 1) * n_kv * geom.v_record_bytes,
                                    dtype=torch.uint8, device=dev) for _ in range(2)]
        ht = np.full(n_pages, -1, np.int32)
        ht[:self.n_hist] = np.arange(self.n_hist, dtype=np.int32)
        self.hist_table = torch.from_numpy(ht).to(dev)
        self.hist_blocks = torch.from_numpy(
            np.tile(np.arange(max(self.n_hist, 1), dtype=np.int32), (n_kv, 1))).to(dev)
        self.hist_pages = list(range(self.n_hist))
        self.splits = kv.kvattn_decode_splits(self.hist_geom, max(self.n_hist, 1))
        rows = n_q_tok * n_kv * geom.gqa
        self.parts = torch.empty((1 + self.splits, rows, kv.HEAD_DIM), dtype=torch.float32,
                                 device=dev)
        self.lparts = torch.empty((1 + self.splits, rows), dtype=torch.float32, device=dev)
        self.ws = torch.empty(workspace_bytes, dtype=torch.uint8, device=dev)
        self.copy = torch.cuda.Stream(device=dev)

    def device_bytes(self):
        """Pool bytes held on the device: resident pools plus staging."""
        res = sum(L.res_k.numel() + L.res_v.numel() for L in self.layers)
        return res + sum(t.numel() for t in self.stage_k + self.stage_v)

    def host_to_device_bytes_per_step(self):
        return sum(self.n_hist * L.res_geom.n_kv_heads *
                   (L.res_geom.k_record_bytes + L.res_geom.v_record_bytes) for L in self.layers)

    def step(self, q, k_new, v_new, kv_len, scale, outs, lses):
        """Enqueue one step over every layer: append the new tokens to the
        resident pool and attend over resident + streamed pages."""
        import torch
        compute = torch.cuda.current_stream()
        n = len(self.layers)
        copied = [torch.cuda.Event() for _ in range(n)]
        done = [torch.cuda.Event() for _ in range(n)]
        for layer in range(n + 1):
            if layer < n and self.n_hist:  # stage layer `layer` once its slot is free
                if layer < 2:
                    self.copy.wait_stream(compute)  # the previous step's last layers
                else:
                    self.copy.wait_event(done[layer - 2])
                L = self.layers[layer]
                kv.kvattn_prefetch_pages(self.hist_geom, L.host_k, L.host_v,
                                         self.stage_k[layer % 2], self.stage_v[layer % 2],
                                         self.hist_pages, stream=self.copy)
                copied[layer].record(self.copy)
            c = layer - 1  # compute the previous layer meanwhile
            if c < 0:
                continue
            L = self.layers[c]
            kv.kvattn_append_decode(L.res_geom, k_new[c], v_new[c], q[c], L.res_k, L.res_v,
                                    L.res_table, kv_len, scale, blocks=L.res_blocks,
                                    out=self.parts[0], lse=self.lparts[0], workspace=self.ws)
            if not self.n_hist:
                outs[c].copy_(self.parts[0].view_as(outs[c]))
                lses[c].copy_(self.lparts[0].view_as(lses[c]))
                continue
            compute.wait_event(copied[c])
            kv.kvattn_decode_partials(self.hist_geom, q[c], self.stage_k[c % 2],
                                      self.stage_v[c % 2], self.hist_table, kv_len, scale,
                                      self.splits, blocks=self.hist_blocks,
                                      o_part=self.parts[1:], lse_part=self.lparts[1:])
            done[c].record(compute)
            kv.kvattn_merge_lse(self.parts, self.lparts, out=outs[c].view(-1, kv.HEAD_DIM),
                                lse=lses[c].view(-1))


class KVMemHostLayer:
    """One layer of KVMem with its history in pinned host memory ([KVMEM]
    測試口徑, "Recall 測試": budget/128 history blocks plus a reserved recent
    window on the GPU, the rest in host RAM). Built from a full device pool:
    every page goes to a pinned host pool (same physical layout), the newest
    n_recent pages stay resident in a compact device pool, and the block
    summaries stay on the device for the selection."""

    def __init__(self, geom, k_pool, v_pool, page_table, n_pages, n_recent, summary):
        import torch
        dev = k_pool.device
        n_kv = geom.n_kv_heads
        self.host_k = torch.empty(k_pool.numel(), dtype=torch.uint8, pin_memory=True)
        self.host_v = torch.empty(v_pool.numel(), dtype=torch.uint8, pin_memory=True)
        self.host_k.copy_(k_pool)
        self.host_v.copy_(v_pool)
        self.recent = StreamedLayer(geom, k_pool, v_pool, page_table, n_pages,
                                    n_pages - min(n_recent, n_pages), keep_history=False)
        self.summary = summary
        torch.cuda.synchronize()


class KVMemHostDecode:
    """Per step and layer: select (kvattn_select_blocks, on the device), pull
    the kept history blocks from host memory (kvattn_gather_blocks: a kernel
    reads the block list on the device and the pages over the host link),
    append + attend over the resident recent window (kvattn_append_decode,
    which also refreshes the summary of a page the append completes), attend
    over the gathered blocks (kvattn_decode_partials) and merge."""

    def __init__(self, geom, layers, page_table, n_pages, n_recent, k_top, n_q_tok, dev,
                 workspace_bytes=64 << 20):
        import torch
        self.geom, self.layers, self.table = geom, layers, page_table
        self.n_pages, self.n_recent, self.k_top = n_pages, n_recent, k_top
        n_kv = geom.n_kv_heads
        r = min(n_recent, n_pages)
        self.k_sel = min(k_top, n_pages - r)
        self.n_out = kv.kvattn_select_count(n_pages, n_recent, k_top)
        self.blocks = torch.empty((n_kv, self.n_out), dtype=torch.int32, device=dev)
        self.sel_ws = torch.empty(8 * n_kv * max(n_pages, 1) + 4096, dtype=torch.uint8, device=dev)
        n_st = max(self.k_sel, 1)
        self.stage_geom = kv.Geom(n_kv, geom.gqa, n_st, v_type=geom.v_type, k_type=geom.k_type)
        self.stage_k = torch.empty(n_st * n_kv * geom.k_record_bytes, dtype=torch.uint8, device=dev)
        self.stage_v = torch.empty(n_st * n_kv * geom.v_record_bytes, dtype=torch.uint8, device=dev)
        self.stage_blocks = torch.empty((n_kv, n_st), dtype=torch.int32, device=dev)
        st = np.full(n_pages, -1, np.int32)
        st[:self.k_sel] = np.arange(self.k_sel, dtype=np.int32)
        self.stage_table = torch.from_numpy(st).to(dev)
        self.splits = kv.kvattn_decode_splits(self.stage_geom, n_st)
        rows = n_q_tok * n_kv * geom.gqa
        self.parts = torch.empty((1 + self.splits, rows, kv.HEAD_DIM), dtype=torch.float32,
                                 device=dev)
        self.lparts = torch.empty((1 + self.splits, rows), dtype=torch.float32, device=dev)
        self.ws = torch.empty(workspace_bytes, dtype=torch.uint8, device=dev)
        self.kept = [torch.empty((n_kv, self.n_out), dtype=torch.int32, device=dev)
                     for _ in layers]

    def host_to_device_bytes_per_step(self):
        return (len(self.layers) * self.k_sel * self.geom.n_kv_heads *
                (self.geom.k_record_bytes + self.geom.v_record_bytes))

    def device_bytes(self):
        res = sum(L.recent.res_k.numel() + L.recent.res_v.numel() + L.summary.numel() * 4
                  for L in self.layers)
        return res + self.stage_k.numel() + self.stage_v.numel()

    def step(self, q, k_new, v_new, kv_len, scale, outs, lses):
        for c, L in enumerate(self.layers):
            kv.kvattn_select_blocks(self.geom, q[c][-1], L.summary, self.n_pages, self.n_pages,
                                    self.n_recent, self.k_top, out_blocks=self.kept[c],
                                    workspace=self.sel_ws)
            R = L.recent
            kv.kvattn_append_decode(R.res_geom, k_new[c], v_new[c], q[c], R.res_k, R.res_v,
                                    R.res_table, kv_len, scale, blocks=R.res_blocks,
                                    k_summary=L.summary, out=self.parts[0], lse=self.lparts[0],
                                    workspace=self.ws)
            if not self.k_sel:
                outs[c].copy_(self.parts[0].view_as(outs[c]))
                lses[c].copy_(self.lparts[0].view_as(lses[c]))
                continue
            kv.kvattn_gather_blocks(self.geom, L.host_k, L.host_v, self.table, self.kept[c],
                                    self.k_sel, self.stage_k, self.stage_v,
                                    dst_blocks=self.stage_blocks)
            kv.kvattn_decode_partials(self.stage_geom, q[c], self.stage_k, self.stage_v,
                                      self.stage_table, kv_len, scale, self.splits,
                                      blocks=self.stage_blocks, o_part=self.parts[1:],
                                      lse_part=self.lparts[1:])
            kv.kvattn_merge_lse(self.parts, self.lparts, out=outs[c].view(-1, kv.HEAD_DIM),
                                lse=lses[c].view(-1))
