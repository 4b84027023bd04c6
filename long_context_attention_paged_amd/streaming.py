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

HostPoolPrefill does the same for chunked prefill ([RDNA4] "Online Log-Sum-Exp
prefill & pipelined prefetch"): every layer's whole pool stays in pinned host
memory as the cache of record, the pages a chunk reads are copied into one of
two device staging pools a layer ahead, the chunk is quantised and attended
there, and the chunk's pages go back to the host pool.
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
        self.ws = kv.workspace(workspace_bytes, dev)
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
        self.sel_ws = kv.workspace(8 * n_kv * max(n_pages, 1) + 4096, dev)
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
        self.ws = kv.workspace(workspace_bytes, dev)
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


class HostPoolPrefill:
    """Chunked prefill with every layer's pool in pinned host memory (a7:
    [RDNA4] "Online Log-Sum-Exp prefill & pipelined prefetch"; [STREAM] step
    ④ prefill with -ub 512 over a host-resident cache). host_k[L], host_v[L]
    are pinned uint8 pools of geom's size (the physical layout of a device
    pool) and page_table the logical-to-physical map shared by the layers.

    Per step and layer, on two streams ordered by events:
     - copy stream: the physical pages of logical pages 0 .. ceil((pos0 +
       chunk) / 128) - 1 go from the host pool to the same slots of one of two
       device staging pools (kvattn_prefetch_pages; layer L+1 copies while
       layer L computes);
     - compute stream: kvattn_quantize_pages writes the chunk's tokens into
       the staged pages, kvattn_prefill_chunk attends;
     - copy stream again: the pages holding the chunk go back to the host pool
       (device to host), so the next chunk reads them there.
    A staging slot is refilled only after its layer's compute and write-back
    are done. Device working set: two staging pools (2 x one layer's pool)."""

    def __init__(self, geom, host_k, host_v, page_table, dev, workspace_bytes=0):
        import torch
        self.geom, self.host_k, self.host_v = geom, host_k, host_v
        self.table = torch.as_tensor(page_table, dtype=torch.int32).to(dev)
        self.table_host = np.asarray(torch.as_tensor(page_table).cpu(), np.int32)
        for t in list(host_k) + list(host_v):
            if not t.is_pinned():
                raise ValueError("HostPoolPrefill needs pinned host pools")
        self.stage_k = [torch.empty(host_k[0].numel(), dtype=torch.uint8, device=dev)
                        for _ in range(2)]
        self.stage_v = [torch.empty(host_v[0].numel(), dtype=torch.uint8, device=dev)
                        for _ in range(2)]
        self.ws = kv.workspace(workspace_bytes, dev)  # grown on demand (zeroed)
        self.dev = dev
        self.copy = torch.cuda.Stream(device=dev)

    def device_bytes(self):
        return sum(t.numel() for t in self.stage_k + self.stage_v)

    def _workspace_for(self, q, pos0):
        need = kv.prefill_workspace_bytes(self.geom, q, self.stage_k[0], self.stage_v[0],
                                          self.table, pos0)
        if self.ws.numel() < need:
            import torch
            torch.cuda.current_stream().synchronize()  # the old one may still be in use
            self.ws = kv.workspace(need, self.dev)

    def pages_read(self, pos0, chunk):
        """Physical pages a chunk at pos0 reads, ascending (so runs coalesce)."""
        n = (pos0 + chunk + PAGE - 1) // PAGE
        return sorted(set(int(x) for x in self.table_host[:n]))

    def pages_written(self, pos0, chunk):
        """Physical pages that hold the chunk's tokens."""
        return sorted(set(int(x) for x in
                          self.table_host[pos0 // PAGE:(pos0 + chunk - 1) // PAGE + 1]))

    def step(self, q, k_new, v_new, pos0, scale, outs, lses):
        """Enqueue one chunk over every layer: q[L] [chunk, n_heads, 256] and
        k_new[L], v_new[L] [chunk, n_kv, 256] (positions pos0 ..), results
        into outs[L], lses[L]."""
        import torch
        compute = torch.cuda.current_stream()
        n = len(q)
        chunk = q[0].shape[0]
        read = self.pages_read(pos0, chunk)
        written = self.pages_written(pos0, chunk)
        self._workspace_for(q[0], pos0)
        copied = [torch.cuda.Event() for _ in range(n)]
        done = [torch.cuda.Event() for _ in range(n)]
        for layer in range(n + 1):
            if layer < n:  # stage layer `layer` once its slot is free
                if layer < 2:
                    self.copy.wait_stream(compute)  # the previous step's last layers
                else:  # its write-back was enqueued before on this stream
                    self.copy.wait_event(done[layer - 2])
                kv.kvattn_prefetch_pages(self.geom, self.host_k[layer], self.host_v[layer],
                                         self.stage_k[layer % 2], self.stage_v[layer % 2],
                                         read, stream=self.copy)
                copied[layer].record(self.copy)
            c = layer - 1  # compute the previous layer meanwhile
            if c < 0:
                continue
            sk, sv = self.stage_k[c % 2], self.stage_v[c % 2]
            compute.wait_event(copied[c])
            kv.kvattn_quantize_pages(self.geom, k_new[c], v_new[c], pos0, self.table, sk, sv)
            kv.kvattn_prefill_chunk(self.geom, q[c], sk, sv, self.table, pos0, scale,
                                    out=outs[c], lse=lses[c], workspace=self.ws)
            done[c].record(compute)
            self.copy.wait_event(done[c])
            kv.kvattn_prefetch_pages(self.geom, sk, sv, self.host_k[c], self.host_v[c], written,
                                     stream=self.copy)
        compute.wait_stream(self.copy)  # the write-backs end the step


def prefill_ranges(pos0, chunk, slot_pages, n_logical_pages):
    """The page ranges [a, b) through which a chunk at pos0 reads its keys
    with staging slots of slot_pages pages: they tile [0, n_read), n_read =
    ceil((pos0 + chunk) / 128), in order, none longer than a slot, and the
    last one ends at n_read and starts at most at pos0's page, so it holds
    every page the chunk writes."""
    n_read = (pos0 + chunk + PAGE - 1) // PAGE
    S = slot_pages
    if n_read - pos0 // PAGE > S:
        raise ValueError(f"the chunk's {n_read - pos0 // PAGE} pages exceed a slot of {S}")
    if n_read > n_logical_pages:
        raise ValueError("the chunk runs past the host tier's pages")
    last = max(0, n_read - S)
    out = [(a, min(a + S, last)) for a in range(0, last, S)]
    return out + [(last, n_read)]


class BudgetedHostPrefill:
    """Chunked prefill from a host tier under a device page budget (the
    Adaptive KV Streaming guide's bounded prefill working set, [STREAM] step
    ④ --kv-resident-mib 450; [RDNA4] "Online Log-Sum-Exp prefill & pipelined
    prefetch"). host_k[L], host_v[L] are pinned pools holding layer L's pages
    in logical page order (page p at record p * n_kv, as StreamedLayer keeps
    its history), so any run of pages is one contiguous copy per pool.

    Two device staging slots of `slot_pages` pages each (budget_bytes / 2 of
    page records) hold page ranges, not whole layers. A chunk at pos0 reads
    logical pages [0, n_read), n_read = ceil((pos0 + chunk) / 128), cut into
    ranges of at most slot_pages pages, the last one ending at n_read (so it
    holds every page the chunk writes). Per (layer, range), in order:
     - copy stream: the range is copied from the host tier into a staging
       slot (kvattn_prefetch_pages: one hipMemcpyAsync per pool), one item
       ahead of the compute;
     - compute: for the last range kvattn_quantize_pages writes the chunk's
       tokens into the staged pages, then kvattn_prefill_range_partials
       attends over that range alone into its share of the partials;
     - after a layer's last range, kvattn_merge_lse combines the ranges'
       partials (the LSE merge is associative over any page split), and the
       staged pages holding the chunk go back to the host tier.
    A slot is refilled only after the compute (and write-back) that read it.
    Device working set: 2 x slot_pages pages, plus the partials."""

    def __init__(self, geom, host_k, host_v, n_logical_pages, dev, budget_bytes):
        import torch
        self.geom, self.host_k, self.host_v, self.dev = geom, host_k, host_v, dev
        self.n_logical = int(n_logical_pages)
        n_kv = geom.n_kv_heads
        self.k_page = n_kv * geom.k_record_bytes
        self.v_page = n_kv * geom.v_record_bytes
        for t in list(host_k) + list(host_v):
            if not t.is_pinned():
                raise ValueError("BudgetedHostPrefill needs pinned host pools")
        for t in host_k:
            if t.numel() < self.n_logical * self.k_page:
                raise ValueError("a host key pool is smaller than n_logical_pages pages")
        for t in host_v:
            if t.numel() < self.n_logical * self.v_page:
                raise ValueError("a host value pool is smaller than n_logical_pages pages")
        self.page_bytes = self.k_page + self.v_page
        self.slot_pages = int(budget_bytes // (2 * self.page_bytes))
        if self.slot_pages < 1:
            raise ValueError("budget too small for two one-page staging slots")
        S = self.slot_pages
        self.stage_geom = kv.Geom(n_kv, geom.gqa, S, v_type=geom.v_type, k_type=geom.k_type)
        self.stage_k = [torch.empty(S * self.k_page, dtype=torch.uint8, device=dev)
                        for _ in range(2)]
        self.stage_v = [torch.empty(S * self.v_page, dtype=torch.uint8, device=dev)
                        for _ in range(2)]
        self.copy = torch.cuda.Stream(device=dev)
        self._plan_key = None

    def device_bytes(self):
        """Staging bytes held on the device (the page budget actually used)."""
        return sum(t.numel() for t in self.stage_k + self.stage_v)

    def ranges(self, pos0, chunk):
        """Logical page ranges [a, b) a chunk at pos0 reads, in order."""
        return prefill_ranges(pos0, chunk, self.slot_pages, self.n_logical)

    def _plan(self, q0, pos0):
        import torch
        chunk = q0.shape[0]
        if self._plan_key == (pos0, chunk):
            return
        rng = self.ranges(pos0, chunk)
        n_read = rng[-1][1]
        g_full = kv.kvattn_prefill_groups(self.stage_geom, chunk, pos0)
        self.plan = []
        first = 0
        for a, b in rng:
            g = max(1, -(-g_full * (b - a) // n_read))  # groups in proportion to the range
            tab = np.full(self.n_logical, -1, np.int32)
            tab[a:b] = np.arange(b - a, dtype=np.int32)
            self.plan.append({"a": a, "b": b, "groups": g, "first": first,
                              "table": torch.from_numpy(tab).to(self.dev),
                              "slots": list(range(b - a)),
                              "geom": kv.Geom(self.geom.n_kv_heads, self.geom.gqa, b - a,
                                              v_type=self.geom.v_type, k_type=self.geom.k_type)})
            first += g
        rows = chunk * self.geom.n_kv_heads * self.geom.gqa
        self.o_parts = torch.empty((first, rows, kv.HEAD_DIM), dtype=torch.float32,
                                   device=self.dev)
        self.lse_parts = torch.empty((first, rows), dtype=torch.float32, device=self.dev)
        a_last = rng[-1][0]
        self.wb_first = pos0 // PAGE                    # the chunk's pages, logical
        self.wb_count = (pos0 + chunk - 1) // PAGE + 1 - self.wb_first
        self.wb_slot = self.wb_first - a_last           # their first slot in the last range
        self._plan_key = (pos0, chunk)

    def host_to_device_bytes_per_step(self, n_layers, pos0, chunk):
        return n_layers * sum(b - a for a, b in self.ranges(pos0, chunk)) * self.page_bytes

    def step(self, q, k_new, v_new, pos0, scale, outs, lses):
        """Enqueue one chunk over every layer: q[L] [chunk, n_heads, 256],
        k_new[L], v_new[L] [chunk, n_kv, 256] (positions pos0 ..), results
        into outs[L], lses[L]."""
        import torch
        compute = torch.cuda.current_stream()
        self._plan(q[0], pos0)
        items = [(L, r) for L in range(len(q)) for r in range(len(self.plan))]
        copied = [torch.cuda.Event() for _ in items]
        done = [torch.cuda.Event() for _ in items]

        def stage(i):
            L, r = items[i]
            pr = self.plan[r]
            a, b = pr["a"], pr["b"]
            if i < 2:
                self.copy.wait_stream(compute)  # the previous step's last items
            else:
                self.copy.wait_event(done[i - 2])  # slot i % 2 has been read
            kv.kvattn_prefetch_pages(
                pr["geom"], self.host_k[L][a * self.k_page:b * self.k_page],
                self.host_v[L][a * self.v_page:b * self.v_page],
                self.stage_k[i % 2], self.stage_v[i % 2], pr["slots"], stream=self.copy)
            copied[i].record(self.copy)

        if items:
            stage(0)
        for i, (L, r) in enumerate(items):
            if i + 1 < len(items):
                stage(i + 1)
            pr = self.plan[r]
            sk, sv = self.stage_k[i % 2], self.stage_v[i % 2]
            compute.wait_event(copied[i])
            last = r == len(self.plan) - 1
            if last:
                kv.kvattn_quantize_pages(self.stage_geom, k_new[L], v_new[L], pos0, pr["table"],
                                         sk, sv)
            g0, g = pr["first"], pr["groups"]
            kv.kvattn_prefill_range_partials(self.stage_geom, q[L], sk, sv, pr["table"], pos0,
                                             scale, pr["a"], pr["b"], g,
                                             o_part=self.o_parts[g0:g0 + g],
                                             lse_part=self.lse_parts[g0:g0 + g])
            done[i].record(compute)
            if last:
                kv.kvattn_merge_lse(self.o_parts, self.lse_parts,
                                    out=outs[L].view(-1, kv.HEAD_DIM), lse=lses[L].view(-1))
                # the chunk's pages back to the host tier (one contiguous run
                # per pool), before the slot is refilled
                self.copy.wait_event(done[i])
                s0, p0, n = self.wb_slot, self.wb_first, self.wb_count
                wb_geom = kv.Geom(self.geom.n_kv_heads, self.geom.gqa, n,
                                  v_type=self.geom.v_type, k_type=self.geom.k_type)
                kv.kvattn_prefetch_pages(
                    wb_geom, sk[s0 * self.k_page:(s0 + n) * self.k_page],
                    sv[s0 * self.v_page:(s0 + n) * self.v_page],
                    self.host_k[L][p0 * self.k_page:(p0 + n) * self.k_page],
                    self.host_v[L][p0 * self.v_page:(p0 + n) * self.v_page],
                    list(range(n)), stream=self.copy)
        compute.wait_stream(self.copy)  # the write-backs end the step
