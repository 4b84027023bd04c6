"""Benchmark of the paged Q8_0/Q4_0 attention hot path on one MI355X.

Headline: decode-attention KV GB/s at 262K context (the verify workload: 16
layers x 4 KV heads x 24 query heads, head_dim 256, 262144 cached tokens, 4
query tokens causal among themselves) and chunked-prefill TFLOP/s (512-token
chunk after 262144 prior tokens), both against the chip's peaks.

A step is one pass over all 16 layers of one workload:
  verify-262k : per layer, one launch that quantises the 4 new tokens into
                their pages and runs decode attention over 2048 pages, then
                the LSE merge;
  prefill-262k: per layer, quantise the 512-token chunk into pages, then
                chunked-prefill attention over 2052 pages with the LSE merge;
  also decode-131k, kvmem-523k (selection + sparse decode), and verify-262k
  with the history streamed from pinned host memory into a 2100 MiB device
  working set (PCIe-bound; never `value`).
Inputs are seeded synthetic tensors (long_context_attention_paged_amd.synth),
resident in HBM before timing; every layer has its own pool so repeated steps
stream from HBM, not from the 256 MB last-level cache. Steps are captured
once in a HIP graph and replayed. Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs 3,4]
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 matrix peak, published
K_REC, V_REC = 34816, 18432
METRIC = "decode-attn KV GB/s (% HBM peak) @262K; prefill-chunk TFLOP/s (% MFMA peak)"
WARM_SECONDS = 0.3             # untimed graph replays before each timed region

# HBM traffic per launch from rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) of `bench.py --profile-kernels`, scaled by what
# the same counters read for a 1 GiB device copy in the same run (FETCH_SIZE
# reads half of the copied bytes, WRITE_SIZE all of them). Valid only for the
# kernel sources and compile flags they were taken on: the sha256 prefixes and
# the flags below are checked at run time and the traffic is reported as null
# once either has changed.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {
    "decode": {"sources": {"decode.hip": "2477d5fb9d026551", "common.hpp": "5e5d1f7f34499a89",
                           "launch.hpp": "525dbebac0e478f8", "qround.hpp": "bfca159575b5ee34"},
               "flags": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "fetch_kib": 213557.85, "write_kib": 6168.0},
    "prefill": {"sources": {"prefill.hip": "12c73f4a90ae4e66", "common.hpp": "5e5d1f7f34499a89",
                            "launch.hpp": "525dbebac0e478f8"},
                "flags": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
                "fetch_kib": 374638.28, "write_kib": 204858.67},
}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the counter runs, or None if its
    sources or compile flags changed since."""
    import hashlib
    from long_context_attention_paged_amd import build
    t = TRAFFIC[kernel]
    if build.EXTRA_FLAGS.get(f"{kernel}.hip", []) != t["flags"]:
        return None
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "long_context_attention_paged_amd", "csrc")
    for name, prefix in t["sources"].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if not hashlib.sha256(f.read()).hexdigest().startswith(prefix):
                return None
    return int(round((t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class LayerPools:
    """One workload's 16 per-layer pools on the GPU plus per-layer queries."""

    def __init__(self, w, dev, with_summary=False, chunk_tokens=32768, v_type=0, k_type=0):
        import torch
        from long_context_attention_paged_amd import synth
        import long_context_attention_paged_amd as kv
        self.w = w
        self.table_np = synth.page_table(w)
        self.table = torch.from_numpy(self.table_np).to(dev)
        self.n_phys = w.n_pages
        self.geom = kv.Geom(w.n_kv, w.gqa, self.n_phys, v_type=v_type, k_type=k_type)
        self.kp, self.vp, self.q, self.summ = [], [], [], []
        self.new_k, self.new_v = [], []
        n_new = w.chunk if w.chunk else w.n_q_tok
        for layer in range(w.n_layers):
            t0 = time.time()
            q = synth.queries(w, layer)
            K, V = synth.kv_layer(w, layer, q, threads=16)
            kp = torch.zeros(self.n_phys * w.n_kv * self.geom.k_record_bytes, dtype=torch.uint8,
                             device=dev)
            vp = torch.zeros(self.n_phys * w.n_kv * self.geom.v_record_bytes, dtype=torch.uint8,
                             device=dev)
            summ = (torch.zeros((w.n_kv, w.n_pages, 256), dtype=torch.float32, device=dev)
                    if with_summary else None)
            for a in range(0, w.kv_len, chunk_tokens):
                b = min(w.kv_len, a + chunk_tokens)
                kv.kvattn_quantize_pages(self.geom, torch.from_numpy(K[a:b]).to(dev),
                                         torch.from_numpy(V[a:b]).to(dev), a, self.table, kp, vp,
                                         summ)
            self.kp.append(kp)
            self.vp.append(vp)
            self.summ.append(summ)
            self.q.append(torch.from_numpy(q).to(dev))
            self.new_k.append(torch.from_numpy(K[w.kv_len - n_new:]).to(dev))
            self.new_v.append(torch.from_numpy(V[w.kv_len - n_new:]).to(dev))
            torch.cuda.synchronize()
            log(f"{w.name}: layer {layer} ready ({time.time() - t0:.1f} s)")


def time_graph(step_fn, steps, warmup):
    """Warm up eagerly (warmup steps), capture one step in a HIP graph, replay it
    untimed for WARM_SECONDS, then time `steps` replays: returns ms/step."""
    import torch
    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step_fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn()
    # untimed replays until the clocks have settled (at least 0.3 s of
    # back-to-back work): a cold GPU runs the first ~30 ms some 4% slower
    t_w = time.perf_counter()
    n = 0
    while n < 2 or time.perf_counter() - t_w < WARM_SECONDS:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, g


MIN_CALLS_PER_GRAPH = 16


def time_launches(call_fn, n_layers, reps):
    """Average duration of one call with HIP events on the stream the work is
    launched on: the n_layers calls (one per layer, so every call reads its own
    pool) are captured back to back in one graph, cycling through the layers
    until the graph holds at least MIN_CALLS_PER_GRAPH calls (so a one-layer
    workload is not timed against the graph's own launch), and a pair of
    events brackets reps replays of it; the figure is the bracketed time over
    the calls replayed (it includes the short gaps between consecutive
    launches)."""
    import torch
    n_calls = max(n_layers, MIN_CALLS_PER_GRAPH)
    for layer in range(n_layers):
        call_fn(layer)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            call_fn(i % n_layers)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * n_calls)


def bench_decode(w, dev, steps, warmup, sparse=False, v_type=0, k_type=0):
    """Decode / verify workload: append the new tokens and attend (one launch), merge (x16).
    v_type 1 caches the values as Q8_0 (272 bytes per token and KV head, as the keys);
    k_type 1 the keys as Q4_0 (144 bytes, as Q4_0 values), k_type 2 as Q5_1 (192 bytes)."""
    import torch
    import long_context_attention_paged_amd as kv
    pools = LayerPools(w, dev, with_summary=sparse, v_type=v_type, k_type=k_type)
    n_out = kv.kvattn_select_count(w.n_pages, w.n_recent, w.k_top) if sparse else 0
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]
    blocks = [torch.empty((w.n_kv, max(n_out, 1)), dtype=torch.int32, device=dev)
              for _ in range(w.n_layers)]
    ws = None

    def decode_call(layer):
        nonlocal ws
        if ws is None:
            ws = kv.workspace(64 << 20, dev)
        kv.kvattn_decode(pools.geom, pools.q[layer], pools.kp[layer], pools.vp[layer],
                         pools.table, w.kv_len, 1.0 / 16.0,
                         blocks=blocks[layer] if sparse else None, out=outs[layer],
                         lse=lses[layer], workspace=ws)

    sel_ws = kv.workspace(8 << 20, dev) if sparse else None
    step_ws = kv.workspace(64 << 20, dev)

    def step():
        # per layer: [select the blocks (kvmem)], then one launch that appends
        # the new tokens to the pool and attends, and the merge (plus the
        # summary of a page the append completes)
        for layer in range(w.n_layers):
            if sparse:
                kv.kvattn_select_blocks(pools.geom, pools.q[layer][-1], pools.summ[layer],
                                        w.n_pages, w.n_pages, w.n_recent, w.k_top,
                                        out_blocks=blocks[layer], workspace=sel_ws)
            kv.kvattn_append_decode(pools.geom, pools.new_k[layer], pools.new_v[layer],
                                    pools.q[layer], pools.kp[layer], pools.vp[layer], pools.table,
                                    w.kv_len, 1.0 / 16.0, blocks=blocks[layer] if sparse else None,
                                    k_summary=pools.summ[layer], out=outs[layer], lse=lses[layer],
                                    workspace=step_ws)

    # the decode kernel alone: the same split-K partials kvattn_decode makes,
    # without its merge
    n_units = blocks[0].shape[1] if sparse else w.n_pages
    n_splits = kv.kvattn_decode_splits(pools.geom, n_units)
    rows = w.n_q_tok * w.n_heads
    o_part = torch.empty((n_splits, rows, 256), dtype=torch.float32, device=dev)
    lse_part = torch.empty((n_splits, rows), dtype=torch.float32, device=dev)

    def kernel_call(layer):
        kv.kvattn_decode_partials(pools.geom, pools.q[layer], pools.kp[layer], pools.vp[layer],
                                  pools.table, w.kv_len, 1.0 / 16.0, n_splits,
                                  blocks=blocks[layer] if sparse else None, o_part=o_part,
                                  lse_part=lse_part)

    ms, _ = time_graph(step, steps, warmup)
    launch_ms = time_launches(decode_call, w.n_layers, max(steps, 3))
    kernel_ms = time_launches(kernel_call, w.n_layers, max(steps, 3))
    tokens = (w.k_top + w.n_recent) * 128 if sparse else w.kv_len
    k_bytes = {kv.K_Q4_0: 144, kv.K_Q5_1: 192}.get(k_type, 272)  # per token and KV head
    bytes_per_launch = tokens * w.n_kv * (k_bytes + (272 if v_type == kv.V_Q8_0 else 144))
    res = {
        "ms_per_step": ms,
        "kv_bytes_per_step": bytes_per_launch * w.n_layers,
        "gbs": bytes_per_launch * w.n_layers / (ms * 1e-3) / 1e9,
        "tokens_per_s": 1e3 / ms,                 # attention-only: one step per token
        "query_tokens_per_s": w.n_q_tok * 1e3 / ms,
        "launch_ms": launch_ms,
        "launch_gbs": bytes_per_launch / (launch_ms * 1e-3) / 1e9,
        "kernel_ms": kernel_ms,
        "kernel_gbs": bytes_per_launch / (kernel_ms * 1e-3) / 1e9,
        "n_splits": n_splits,
        "bytes_per_launch": bytes_per_launch,
    }
    if sparse:
        res["recall"] = needle_recall(w, pools, blocks)
        pools.blocks0 = blocks[0]  # layer 0's selection, for the CPU baseline
    return res, pools


def rotation_quality(w, pools, dev):
    """Key rotation on the decode workload's outlier channels: layer 0's cache
    rebuilt from Hadamard-rotated keys (kvattn_rotate_rows before
    kvattn_quantize_pages, the query rotated too) against the plain cache, both
    compared with exact binary64 attention over the unquantised keys and values
    for the 6 query rows of KV head 0 (numpy here, not the oracle)."""
    import numpy as np
    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import synth
    q_np = synth.queries(w, 0)
    K, V = synth.kv_layer(w, 0, q_np, threads=16)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    kv.kvattn_rotate_rows(Kd)
    kr = torch.zeros_like(pools.kp[0])
    vr = torch.zeros_like(pools.vp[0])
    kv.kvattn_quantize_pages(pools.geom, Kd, Vd, 0, pools.table, kr, vr)
    qr = pools.q[0].clone()
    kv.kvattn_rotate_rows(qr)
    out_r, _ = kv.kvattn_decode(pools.geom, qr, kr, vr, pools.table, w.kv_len, 1.0 / 16.0)
    out_p, _ = kv.kvattn_decode(pools.geom, pools.q[0], pools.kp[0], pools.vp[0], pools.table,
                                w.kv_len, 1.0 / 16.0)
    # values rotated too: H/16 is symmetric and orthonormal, so rotating the
    # output rows once more undoes it (o = R sum p R v)
    kv.kvattn_rotate_rows(Vd)
    kvv = torch.zeros_like(pools.kp[0])
    vvv = torch.zeros_like(pools.vp[0])
    kv.kvattn_quantize_pages(pools.geom, Kd, Vd, 0, pools.table, kvv, vvv)
    out_kv, _ = kv.kvattn_decode(pools.geom, qr, kvv, vvv, pools.table, w.kv_len, 1.0 / 16.0)
    kv.kvattn_rotate_rows(out_kv)
    rows = q_np[0, :w.gqa].astype(np.float64)            # query heads of KV head 0
    s = rows @ K[:, 0].astype(np.float64).T / 16.0
    p = np.exp(s - s.max(axis=1, keepdims=True))
    exact = (p @ V[:, 0].astype(np.float64)) / p.sum(axis=1, keepdims=True)
    res = {"sample": "decode-131k layer 0, KV head 0, 6 query rows, 4 channels x8 (keys and "
                     "values); scores isolate the key error, outputs include the values'"}

    def head0_keys(pool):
        # dequantised keys of KV head 0 in token order, from the pool's layout
        rec = pool.view(-1, w.n_kv, K_REC)[pools.table.long(), 0].cpu().numpy()
        codes = rec[:, :32768].view(np.int8).reshape(-1, 128, 8, 32).astype(np.float64)
        d = rec[:, 32768:].view(np.float16).reshape(-1, 128, 8, 1).astype(np.float64)
        return (codes * d).reshape(-1, 256)[:w.kv_len]

    qrot = qr[0, :w.gqa].double().cpu().numpy()
    for name, out, pool, qrows in (("plain", out_p, pools.kp[0], rows),
                                   ("rotated_k", out_r, kr, qrot),
                                   ("rotated_kv", out_kv, None, None)):
        o = out[0, :w.gqa].double().cpu().numpy()
        res[f"out_max_abs_err_{name}"] = float(np.abs(o - exact).max())
        res[f"out_rel_rms_err_{name}"] = float(np.sqrt(((o - exact) ** 2).sum() / (exact ** 2).sum()))
        if pool is not None:
            s_hat = qrows @ head0_keys(pool).T / 16.0
            res[f"score_rel_rms_err_{name}"] = float(
                np.sqrt(((s_hat - s) ** 2).sum() / (s ** 2).sum()))
    del Kd, Vd, kr, vr, kvv, vvv
    torch.cuda.empty_cache()
    return res


def needle_recall(w, pools, blocks):
    from long_context_attention_paged_amd import synth
    needles = set(int(b) for b in synth.needle_blocks(w))
    hits = []
    for layer in range(w.n_layers):
        b = blocks[layer].cpu().numpy()
        for h in range(w.n_kv):
            hits.append(len(needles & set(b[h].tolist())))
    return {"needles": len(needles), "min_found": min(hits), "mean_found": sum(hits) / len(hits)}


def recall_curve(dev, n_layers=2, contexts=(131072, 262144, 393216, 523264),
                 budgets=(32768, 65536, 98304), per_block=3):
    """Needle recall of the selection against context length and budget, with
    faint needles (synth.faint_needle_keys: `per_block` needle tokens in each
    of 20 needle blocks, all within the first 112K tokens so every context
    holds them). The keys of the longest context are quantised once per layer
    (with their block summaries); a shorter context selects over the prefix of
    its blocks (its own recent window of 128 blocks, k_top = budget / 128).
    Recall = needle blocks kept, over every (layer, KV head)."""
    import numpy as np
    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import synth
    w = synth.WORKLOADS[5]
    n_pages = w.n_pages
    span = min(contexts) // 128 - w.n_recent
    geom = kv.Geom(w.n_kv, w.gqa, n_pages)
    table = torch.arange(n_pages, dtype=torch.int32, device=dev)
    kp = torch.zeros(n_pages * w.n_kv * geom.k_record_bytes, dtype=torch.uint8, device=dev)
    vp = torch.zeros(n_pages * w.n_kv * geom.v_record_bytes, dtype=torch.uint8, device=dev)
    summ = torch.zeros((w.n_kv, n_pages, 256), dtype=torch.float32, device=dev)
    ws = kv.workspace(8 * w.n_kv * n_pages + 4096, dev)
    points = [(c, 32768) for c in contexts] + [(contexts[-1], b) for b in budgets if b != 32768]
    found = {p: [] for p in points}
    for layer in range(n_layers):
        q = synth.queries(w, layer)
        K = np.empty((w.kv_len, w.n_kv, 256), np.float32)
        needles = None
        for h in range(w.n_kv):
            K[:, h], needles = synth.faint_needle_keys(w, layer, h, q, span, per_block)
        step = 65536
        zeros = torch.zeros((step, w.n_kv, 256), dtype=torch.float32, device=dev)
        for a in range(0, w.kv_len, step):
            b = min(w.kv_len, a + step)
            kv.kvattn_quantize_pages(geom, torch.from_numpy(K[a:b]).to(dev), zeros[:b - a], a,
                                     table, kp, vp, summ)
        del K
        qd = torch.from_numpy(q[-1]).to(dev)
        nset = set(int(x) for x in needles)
        for ctx, budget in points:
            nb = ctx // 128
            out = torch.empty((w.n_kv, kv.kvattn_select_count(nb, w.n_recent, budget // 128)),
                              dtype=torch.int32, device=dev)
            kv.kvattn_select_blocks(geom, qd, summ, n_pages, nb, w.n_recent, budget // 128,
                                    out_blocks=out, workspace=ws)
            sel = out.cpu().numpy()
            for h in range(w.n_kv):
                found[(ctx, budget)].append(len(nset & set(sel[h].tolist())))
    return {
        "needle_model": f"{per_block} needle tokens (cosine 1/2 to the query group's sum) in each "
                        f"of {w.n_needles} blocks among the first {span} blocks, N(0,1) keys "
                        f"otherwise; {n_layers} layers x {w.n_kv} KV heads",
        "points": [{"context": ctx, "budget": budget, "k_top": budget // 128,
                    "candidates": ctx // 128 - w.n_recent,
                    "mean_found": float(np.mean(found[(ctx, budget)])),
                    "min_found": int(np.min(found[(ctx, budget)])),
                    "max_found": int(np.max(found[(ctx, budget)])), "of": w.n_needles}
                   for ctx, budget in points],
    }


def prefill_flops_per_layer(w):
    """4 * D flops per unmasked (query head, key) pair, one layer."""
    pairs = w.chunk * w.pos0 + w.chunk * (w.chunk + 1) // 2
    return 4 * 256 * pairs * w.n_heads


def bench_prefill(w, dev, steps, warmup, v_type=0, k_type=0):
    import torch
    import long_context_attention_paged_amd as kv
    pools = LayerPools(w, dev, v_type=v_type, k_type=k_type)
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]
    ws = kv.workspace(512 << 20, dev)

    def prefill_call(layer):
        kv.kvattn_prefill_chunk(pools.geom, pools.q[layer], pools.kp[layer], pools.vp[layer],
                                pools.table, w.pos0, 1.0 / 16.0, out=outs[layer],
                                lse=lses[layer], workspace=ws)

    def step():
        for layer in range(w.n_layers):
            kv.kvattn_quantize_pages(pools.geom, pools.new_k[layer], pools.new_v[layer], w.pos0,
                                     pools.table, pools.kp[layer], pools.vp[layer])
            prefill_call(layer)

    # the prefill kernel alone: kvattn_prefill_chunk's per-group partials
    n_groups = kv.kvattn_prefill_groups(pools.geom, w.chunk, w.pos0)
    rows = w.chunk * w.n_heads
    o_part = torch.empty((n_groups, rows, 256), dtype=torch.float32, device=dev)
    lse_part = torch.empty((n_groups, rows), dtype=torch.float32, device=dev)

    def kernel_call(layer):
        kv.kvattn_prefill_partials(pools.geom, pools.q[layer], pools.kp[layer], pools.vp[layer],
                                   pools.table, w.pos0, 1.0 / 16.0, n_groups, o_part=o_part,
                                   lse_part=lse_part)

    ms, _ = time_graph(step, steps, warmup)
    reps = max(2, min(steps, 3))
    launch_ms = time_launches(prefill_call, w.n_layers, reps)
    kernel_ms = time_launches(kernel_call, w.n_layers, reps)
    fl = prefill_flops_per_layer(w)
    return {
        "ms_per_step": ms,
        "flops_per_step": fl * w.n_layers,
        "tflops": fl * w.n_layers / (ms * 1e-3) / 1e12,
        "tokens_per_s": w.chunk / (ms * 1e-3),
        "launch_ms": launch_ms,
        "flops_per_launch": fl,
        "launch_tflops": fl / (launch_ms * 1e-3) / 1e12,
        "kernel_ms": kernel_ms,
        "kernel_tflops": fl / (kernel_ms * 1e-3) / 1e12,
        "n_groups": n_groups,
    }, pools


def bench_prefill_host_pool(w, dev, steps, warmup):
    """Prefill with every layer's pool in pinned host memory (a7,
    streaming.HostPoolPrefill): while layer L computes from one device staging
    pool, a copy stream fills the other with layer L+1's pages, and each
    layer's chunk pages go back to the host pool. Bound by the host link, not
    by the GPU."""
    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import streaming
    pools = LayerPools(w, dev)
    hk, hv = [], []
    for layer in range(w.n_layers):  # move every layer's pool to pinned host memory
        hk.append(torch.empty(pools.kp[layer].numel(), dtype=torch.uint8, pin_memory=True))
        hv.append(torch.empty(pools.vp[layer].numel(), dtype=torch.uint8, pin_memory=True))
        hk[layer].copy_(pools.kp[layer])
        hv[layer].copy_(pools.vp[layer])
    torch.cuda.synchronize()
    pools.kp = pools.vp = None
    torch.cuda.empty_cache()
    hp = streaming.HostPoolPrefill(pools.geom, hk, hv, pools.table, dev)
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]

    def step():
        hp.step(pools.q, pools.new_k, pools.new_v, w.pos0, 1.0 / 16.0, outs, lses)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    fl = prefill_flops_per_layer(w)
    geom = pools.geom
    page = geom.n_kv_heads * (geom.k_record_bytes + geom.v_record_bytes)
    h2d = len(hp.pages_read(w.pos0, w.chunk)) * page * w.n_layers
    d2h = len(hp.pages_written(w.pos0, w.chunk)) * page * w.n_layers
    return {
        "ms_per_step": ms,
        "tokens_per_s": w.chunk / (ms * 1e-3),
        "tflops": fl * w.n_layers / (ms * 1e-3) / 1e12,
        "host_to_device_bytes_per_step": h2d,
        "host_to_device_gbs": h2d / (ms * 1e-3) / 1e9,
        "device_to_host_bytes_per_step": d2h,
        "device_pool_bytes": hp.device_bytes(),
        "workspace_error": kv.workspace_error(hp.ws),
        "note": "pools in pinned host memory, layer-ahead page prefetch on a copy stream, "
                "chunk pages written back",
    }, pools


def bench_prefill_budgeted(w, dev, steps, warmup, budget=450 << 20):
    """Prefill with every layer's pool in pinned host memory and a bounded
    device working set (streaming.BudgetedHostPrefill; the Adaptive KV
    Streaming guide's --kv-resident-mib 450): each layer's pages pass through
    two staging slots of budget / 2 in page ranges, one range ahead of the
    compute, and the ranges' partials are merged by LSE. Bound by the host
    link."""
    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import streaming
    pools = LayerPools(w, dev)
    hk, hv = [], []
    tl = pools.table.long()
    for layer in range(w.n_layers):  # each layer's pages to a host tier in logical order
        kview = pools.kp[layer].view(pools.n_phys, -1)
        vview = pools.vp[layer].view(pools.n_phys, -1)
        hk.append(torch.empty(w.n_pages * kview.shape[1], dtype=torch.uint8, pin_memory=True))
        hv.append(torch.empty(w.n_pages * vview.shape[1], dtype=torch.uint8, pin_memory=True))
        hk[layer].copy_(kview[tl].reshape(-1))
        hv[layer].copy_(vview[tl].reshape(-1))
        torch.cuda.synchronize()
    pools.kp = pools.vp = None
    torch.cuda.empty_cache()
    bp = streaming.BudgetedHostPrefill(pools.geom, hk, hv, w.n_pages, dev, budget)
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]

    def step():
        bp.step(pools.q, pools.new_k, pools.new_v, w.pos0, 1.0 / 16.0, outs, lses)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    fl = prefill_flops_per_layer(w)
    h2d = bp.host_to_device_bytes_per_step(w.n_layers, w.pos0, w.chunk)
    return {
        "ms_per_step": ms,
        "tokens_per_s": w.chunk / (ms * 1e-3),
        "tflops": fl * w.n_layers / (ms * 1e-3) / 1e12,
        "device_budget_bytes": budget,
        "device_pool_bytes": bp.device_bytes(),
        "ranges_per_layer": len(bp.ranges(w.pos0, w.chunk)),
        "host_to_device_bytes_per_step": h2d,
        "host_to_device_gbs": h2d / (ms * 1e-3) / 1e9,
        "note": "pages in a pinned host tier (logical order), page ranges copied into two "
                "budget/2 staging slots one range ahead, range partials merged by LSE",
    }, pools


def bench_verify_streamed(w, dev, steps, warmup, budget=2100 << 20):
    """Verify with adaptive host-resident KV streaming: a device working set of
    `budget` bytes (the pages' decode figure, 2100 MiB) holds each layer's
    newest pages plus two staging pools; every step streams each layer's older
    history from pinned host memory over PCIe while the previous layer
    computes, appends the 4 new tokens to the resident pages, attends over
    both tiers and merges them. Bound by the host link, not by the GPU."""
    import torch
    from long_context_attention_paged_amd import streaming
    pools = LayerPools(w, dev)
    n_res = streaming.resident_pages_for_budget(budget, w.n_layers, w.n_pages, w.n_kv)
    n_hist = w.n_pages - n_res
    layers = []
    for layer in range(w.n_layers):  # full device pool -> host history + resident pages
        layers.append(streaming.StreamedLayer(pools.geom, pools.kp[layer], pools.vp[layer],
                                              pools.table, w.n_pages, n_hist))
        pools.kp[layer] = pools.vp[layer] = None
    torch.cuda.empty_cache()
    sd = streaming.StreamedDecode(pools.geom, layers, w.n_pages, w.n_q_tok, dev)
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]

    def step():
        sd.step(pools.q, pools.new_k, pools.new_v, w.kv_len, 1.0 / 16.0, outs, lses)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    h2d = sd.host_to_device_bytes_per_step()
    kv_bytes = w.kv_len * w.n_kv * (272 + 144) * w.n_layers
    return {
        "ms_per_step": ms,
        "tokens_per_s": 1e3 / ms,
        "query_tokens_per_s": w.n_q_tok * 1e3 / ms,
        "gbs": kv_bytes / (ms * 1e-3) / 1e9,
        "device_budget_bytes": budget,
        "device_pool_bytes": sd.device_bytes(),
        "resident_pages_per_layer": n_res,
        "streamed_pages_per_layer": n_hist,
        "host_to_device_bytes_per_step": h2d,
        "host_to_device_gbs": h2d / (ms * 1e-3) / 1e9,
        "note": "history in pinned host memory, newest pages resident, layer-ahead staging",
    }, pools


def bench_kvmem_host(w, dev, steps, warmup, budgets=(32768, 65536, 98304)):
    """KVMem with the history in pinned host memory: per step and layer the
    blocks selected on the device are pulled over the host link by a kernel
    (kvattn_gather_blocks) and attended with the resident recent window. For
    each token budget (k_top = budget / 128 history blocks): step time, the
    needle recall of the selection, and the share of full attention's softmax
    mass the kept blocks carry (exp(lse_sparse - lse_full) per row)."""
    import numpy as np
    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import streaming
    pools = LayerPools(w, dev, with_summary=True)
    ws = kv.workspace(64 << 20, dev)
    lse_full = []
    for layer in range(w.n_layers):  # full attention (with this step's append) for the coverage
        o = torch.empty_like(pools.q[layer])
        l_ = torch.empty(pools.q[layer].shape[:2], dtype=torch.float32, device=dev)
        kv.kvattn_append_decode(pools.geom, pools.new_k[layer], pools.new_v[layer],
                                pools.q[layer], pools.kp[layer], pools.vp[layer], pools.table,
                                w.kv_len, 1.0 / 16.0, out=o, lse=l_, workspace=ws)
        lse_full.append(l_)
    layers = []
    for layer in range(w.n_layers):
        layers.append(streaming.KVMemHostLayer(pools.geom, pools.kp[layer], pools.vp[layer],
                                               pools.table, w.n_pages, w.n_recent,
                                               pools.summ[layer]))
        pools.kp[layer] = pools.vp[layer] = None
    torch.cuda.empty_cache()
    outs = [torch.empty_like(q) for q in pools.q]
    lses = [torch.empty(q.shape[:2], dtype=torch.float32, device=dev) for q in pools.q]
    res = {"note": "history in pinned host memory, kept blocks gathered by kernel over the host "
                   "link, recent window resident", "budgets": {}}
    for budget in budgets:
        k_top = budget // 128
        kd = streaming.KVMemHostDecode(pools.geom, layers, pools.table, w.n_pages, w.n_recent,
                                       k_top, w.n_q_tok, dev)

        def step():
            kd.step(pools.q, pools.new_k, pools.new_v, w.kv_len, 1.0 / 16.0, outs, lses)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        cover = torch.cat([torch.exp(lses[c] - lse_full[c]).reshape(-1)
                           for c in range(w.n_layers)])
        h2d = kd.host_to_device_bytes_per_step()
        tokens = (kd.k_sel + min(w.n_recent, w.n_pages)) * 128
        res["budgets"][str(budget)] = {
            "k_top": k_top,
            "ms_per_step": ms,
            "tokens_per_s": 1e3 / ms,
            "attended_tokens": tokens,
            "kv_gbs": tokens * w.n_kv * (272 + 144) * w.n_layers / (ms * 1e-3) / 1e9,
            "host_to_device_bytes_per_step": h2d,
            "host_to_device_gbs": h2d / (ms * 1e-3) / 1e9,
            "device_pool_bytes": kd.device_bytes(),
            "recall": needle_recall(w, pools, kd.kept),
            "mass_covered": {"mean": float(cover.mean()), "min": float(cover.min())},
        }
        log(f"{w.name} host tier, budget {budget}: {json.dumps(res['budgets'][str(budget)])}")
        del kd
    return res, pools


def cpu_baseline_decode(w, pools, blocks=None):
    """The oracle, as it stands, on layer 0 of the workload (every KV head;
    with `blocks`, layer 0's selected block lists: the sparse decode)."""
    import oracle
    kp = pools.kp[0].cpu().numpy().reshape(pools.n_phys, w.n_kv, K_REC)
    vp = pools.vp[0].cpu().numpy().reshape(pools.n_phys, w.n_kv, V_REC)
    q = pools.q[0].cpu().numpy()
    blk = None if blocks is None else blocks.cpu().numpy()
    t0 = time.perf_counter()
    oracle.decode(q, w.gqa, kp, vp, pools.table_np, w.n_pages, w.kv_len, 1.0 / 16.0,
                  blocks=blk)
    dt = time.perf_counter() - t0
    tokens = w.kv_len if blk is None else blk.shape[1] * 128
    nbytes = tokens * w.n_kv * (272 + 144)
    what = (f"{tokens} tokens" if blk is None else
            f"the {blk.shape[1]} selected blocks ({tokens} tokens)")
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": dt,
            "sample": f"{w.name}: layer 0 of {w.n_layers}, all {w.n_kv} KV heads ({what} x "
                      f"{w.gqa * w.n_q_tok} query rows per KV head), binary64, numpy + OpenBLAS"}


def cpu_baseline_prefill(w, pools, n_tok=24):
    import numpy as np
    import oracle
    kp = pools.kp[0].cpu().numpy().reshape(pools.n_phys, w.n_kv, K_REC)
    vp = pools.vp[0].cpu().numpy().reshape(pools.n_phys, w.n_kv, V_REC)
    q = pools.q[0].cpu().numpy()
    toks = np.linspace(0, w.chunk - 1, n_tok).astype(np.int64)
    t0 = time.perf_counter()
    oracle.prefill_chunk(q, w.gqa, kp, vp, pools.table_np, w.n_pages, w.pos0, 1.0 / 16.0,
                         tokens=toks, kv_heads=[0])
    dt = time.perf_counter() - t0
    fl = 4 * 256 * w.gqa * int(sum(w.pos0 + t + 1 for t in toks))
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": dt,
            "sample": f"{w.name}: layer 0, KV head 0, {n_tok} of {w.chunk} query tokens "
                      f"({n_tok * w.gqa} rows over {w.kv_len} keys), binary64, numpy + OpenBLAS"}


def cpu_baseline_tiny_one_thread():
    """The oracle on the tiny decode workload (one layer, one KV head, 4096
    tokens, identity table, one query) with one BLAS thread; its pages are
    quantised by the oracle too, so no device is involved."""
    import numpy as np
    import oracle
    from oracle import quant
    from threadpoolctl import threadpool_limits
    from long_context_attention_paged_amd import synth
    w = synth.WORKLOADS[1]
    q = synth.queries(w, 0)
    K, V = synth.kv_layer(w, 0, q, threads=1)
    table = synth.page_table(w)
    kp = np.zeros((w.n_pages, w.n_kv, K_REC), np.uint8)
    vp = np.zeros((w.n_pages, w.n_kv, V_REC), np.uint8)
    quant.quantize_into_pool(K, V, 0, table, kp, vp)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        reps = 0
        while reps < 3 or time.perf_counter() - t0 < 1.0:
            oracle.decode(q, w.gqa, kp, vp, table, w.n_pages, w.kv_len, 1.0 / 16.0)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    nbytes = w.kv_len * w.n_kv * (272 + 144)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds_per_call": dt,
            "sample": f"{w.name}: the whole workload ({w.kv_len} tokens x {w.gqa} query rows), "
                      "binary64, numpy + OpenBLAS, one thread"}


def gemm_probe(dev, n=8192, reps=20):
    """Dense f16 matrix-core rate of the vendor library on this GPU: torch.mm of
    two contiguous n x n f16 matrices (hipBLASLt), fp32 accumulate inside."""
    import torch
    a = torch.randn(n, n, dtype=torch.float16, device=dev)
    b = torch.randn(n, n, dtype=torch.float16, device=dev)
    c = torch.empty(n, n, dtype=torch.float16, device=dev)
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < WARM_SECONDS:
        torch.mm(a, b, out=c)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"tflops": round(tflops, 1), "frac_of_published_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "what": f"torch.mm f16 {n}x{n}x{n} (hipBLASLt), {reps} calls"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model /
    stepping, clock and the logical CPUs this process may run on."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                info.setdefault(k.strip(), v.strip())
    except OSError:
        return platform.processor()
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return (f"{info.get('model name', platform.processor())} (family {info.get('cpu family', '?')}"
            f" model {info.get('model', '?')} stepping {info.get('stepping', '?')}, "
            f"{info.get('cpu MHz', '?')} MHz, {info.get('cpu cores', '?')} cores per socket, "
            f"{usable} logical CPUs usable)")


def profile_kernels(dev, layers, reps):
    """A short fixed sequence for counter runs (rocprofv3 --pmc): a device copy
    of 1 GiB (the calibration kernel: reads and writes exactly 1 GiB), then the
    decode kernel on verify-262k (Q8_0 keys, then Q4_0 and Q5_1 keys) and the
    prefill kernel on prefill-512-after-262k, each over `layers` per-layer
    pools, `reps` times."""
    import torch
    import long_context_attention_paged_amd as kv
    from dataclasses import replace
    from long_context_attention_paged_amd import synth
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log(f"profile: copied {n} bytes x {reps}")
    w = replace(synth.WORKLOADS[3], n_layers=layers)
    pools = LayerPools(w, dev)
    S = kv.kvattn_decode_splits(pools.geom, w.n_pages)
    o_part = torch.empty((S, w.n_q_tok * w.n_heads, 256), dtype=torch.float32, device=dev)
    lse_part = torch.empty((S, w.n_q_tok * w.n_heads), dtype=torch.float32, device=dev)
    for _ in range(reps):
        for layer in range(layers):
            kv.kvattn_decode_partials(pools.geom, pools.q[layer], pools.kp[layer],
                                      pools.vp[layer], pools.table, w.kv_len, 1.0 / 16.0, S,
                                      o_part=o_part, lse_part=lse_part)
    torch.cuda.synchronize()
    log(f"profile: decode_kernel x {reps * layers}, {w.kv_len * w.n_kv * 416} KV bytes each")
    del pools
    # the nibble-key pairs (q4_0/q4_0, q5_1/q4_0): the same launches
    for k_type, k_bytes in ((kv.K_Q4_0, 144), (kv.K_Q5_1, 192)):
        pools = LayerPools(w, dev, k_type=k_type)
        for _ in range(reps):
            for layer in range(layers):
                kv.kvattn_decode_partials(pools.geom, pools.q[layer], pools.kp[layer],
                                          pools.vp[layer], pools.table, w.kv_len, 1.0 / 16.0, S,
                                          o_part=o_part, lse_part=lse_part)
        torch.cuda.synchronize()
        log(f"profile: decode_kernel (key type {k_type}) x {reps * layers}, "
            f"{w.kv_len * w.n_kv * (k_bytes + 144)} KV bytes each")
        del pools
    del o_part, lse_part
    torch.cuda.empty_cache()
    w = replace(synth.WORKLOADS[4], n_layers=layers)
    pools = LayerPools(w, dev)
    G = kv.kvattn_prefill_groups(pools.geom, w.chunk, w.pos0)
    o_part = torch.empty((G, w.chunk * w.n_heads, 256), dtype=torch.float32, device=dev)
    lse_part = torch.empty((G, w.chunk * w.n_heads), dtype=torch.float32, device=dev)
    for _ in range(reps):
        for layer in range(layers):
            kv.kvattn_prefill_partials(pools.geom, pools.q[layer], pools.kp[layer],
                                       pools.vp[layer], pools.table, w.pos0, 1.0 / 16.0, G,
                                       o_part=o_part, lse_part=lse_part)
    torch.cuda.synchronize()
    log(f"profile: prefill_kernel x {reps * layers}, {prefill_flops_per_layer(w)} flop each")


# bench config -> (k_type, v_type, tag) of the other KV cache type pairs
PAIRS = {"3q8": (0, 1, "q8_0-q8_0"), "4q8": (0, 1, "q8_0-q8_0"),
         "3q4": (1, 0, "q4_0-q4_0"), "4q4": (1, 0, "q4_0-q4_0"),
         "3q5": (2, 0, "q5_1-q4_0"), "4q5": (2, 0, "q5_1-q4_0")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default="3,4,2,5,1,3s,5h,4b,3q4,3q5",
                    help="workloads to run: 1 tiny-decode-4k (latency), 2 decode-131k, "
                         "3 verify-262k, 4 prefill, 5 kvmem, "
                         "4h prefill with the pool in pinned host memory (whole layers "
                         "staged), 4b the same under a 450 MiB device budget (page ranges), "
                         "3s verify with the "
                         "history streamed from host memory (2100 MiB device working set), "
                         "5h kvmem with its history in host memory (budget sweep), "
                         "3q8 / 4q8 verify-262k / prefill with the q8_0/q8_0 pair, "
                         "3q4 / 4q4 with the q4_0/q4_0 pair, 3q5 / 4q5 with q5_1/q4_0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="run only a short fixed kernel sequence for counter runs (no JSON line)")
    ap.add_argument("--layers", type=int, default=2, help="pools per workload in --profile-kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_attention_paged_amd as kv
    from long_context_attention_paged_amd import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    kv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_kernels:
        profile_kernels(dev, args.layers, max(1, args.steps))
        return
    cfgs = [c.strip() for c in args.configs.split(",") if c.strip()]
    extra = {}
    decode_res = prefill_res = None
    cpu = None
    for c in cfgs:
        if c == "5h":
            w = synth.WORKLOADS[5]
            log(f"workload {w.name} (host tier)")
            res, pools = bench_kvmem_host(w, dev, max(2, min(args.steps, 5)), 1)
            extra[w.name + "-host-tier"] = res
            del pools
            torch.cuda.empty_cache()
            continue
        if c == "3s":
            w = synth.WORKLOADS[3]
            log(f"workload {w.name} (streamed history)")
            res, pools = bench_verify_streamed(w, dev, max(2, min(args.steps, 5)), 1)
            extra[w.name + "-streamed"] = res
            del pools
            torch.cuda.empty_cache()
            log(f"{w.name} streamed: {json.dumps(res)}")
            continue
        if c in PAIRS:  # the other cache type pairs: q8_0/q8_0, q4_0/q4_0
            k_type, v_type, tag = PAIRS[c]
            w = synth.WORKLOADS[int(c[0])]
            log(f"workload {w.name} ({tag})")
            fn = bench_decode if c[0] == "3" else bench_prefill
            res, pools = fn(w, dev, args.steps, args.warmup, v_type=v_type, k_type=k_type)
            extra[f"{w.name}-{tag}"] = res
            del pools
            torch.cuda.empty_cache()
            log(f"{w.name} {tag}: {json.dumps(res)}")
            continue
        if c == "4b":
            w = synth.WORKLOADS[4]
            log(f"workload {w.name} (host pool, 450 MiB device budget)")
            res, pools = bench_prefill_budgeted(w, dev, max(2, min(args.steps, 5)), 1)
            extra[w.name + "-host-budget-450mib"] = res
            del pools
            torch.cuda.empty_cache()
            log(f"{w.name} host pool, budget: {json.dumps(res)}")
            continue
        if c == "4h":
            w = synth.WORKLOADS[4]
            log(f"workload {w.name} (host pool)")
            res, pools = bench_prefill_host_pool(w, dev, max(2, min(args.steps, 5)), 1)
            extra[w.name + "-host-pool"] = res
            del pools
            torch.cuda.empty_cache()
            log(f"{w.name} host pool: {json.dumps(res)}")
            continue
        c = int(c)
        w = synth.WORKLOADS[c]
        log(f"workload {w.name}")
        if c in (1, 2, 3):
            res, pools = bench_decode(w, dev, args.steps, args.warmup)
            if c == 1:  # a latency case: one small layer per step
                res["us_per_step"] = res["ms_per_step"] * 1e3
                res["kernel_us"] = res["kernel_ms"] * 1e3
                res["call_us"] = res["launch_ms"] * 1e3
            if c == 2:
                res["key_rotation"] = rotation_quality(w, pools, dev)
                if not args.no_cpu_baseline:
                    res["cpu_baseline"] = cpu_baseline_decode(w, pools)
            if c == 3:
                decode_res = res
                if not args.no_cpu_baseline:
                    cpu = cpu_baseline_decode(w, pools)
            extra[w.name] = res
        elif c == 4:
            res, pools = bench_prefill(w, dev, args.steps, args.warmup)
            prefill_res = res
            if not args.no_cpu_baseline:
                res["cpu_baseline"] = cpu_baseline_prefill(w, pools)
            extra[w.name] = res
        elif c == 5:
            res, pools = bench_decode(w, dev, args.steps, args.warmup, sparse=True)
            if not args.no_cpu_baseline:
                res["cpu_baseline"] = cpu_baseline_decode(w, pools, blocks=pools.blocks0)
            extra[w.name] = res
            del pools
            torch.cuda.empty_cache()
            pools = None
            res["recall_curve"] = recall_curve(dev)
            log(f"{w.name} recall curve: {json.dumps(res['recall_curve'])}")
        del pools
        torch.cuda.empty_cache()
        log(f"{w.name}: {json.dumps(res)}")

    head = decode_res or next((v for v in extra.values() if "ms_per_step" in v),
                              {"ms_per_step": 0.0})
    w3 = synth.WORKLOADS[3]
    line = {
        "metric": METRIC,
        "value": round(head.get("gbs", 0.0), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "verify-262k: 16 layers x 4 KV heads x 24 query heads (GQA 6), head_dim 256, "
                        "262144 cached tokens in 2048 128-token pages (seeded permutation), "
                        "4 query tokens causal among themselves, Q8_0 K / Q4_0 V, N(0,1)",
            "layers": w3.n_layers, "kv_heads": w3.n_kv, "q_heads": w3.n_heads,
            "head_dim": 256, "context": w3.kv_len, "query_tokens": w3.n_q_tok,
        },
        "hbm_frac": round(head.get("gbs", 0.0) / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(head.get("tokens_per_s", 0.0), 1),
        "query_tokens_per_s": round(head.get("query_tokens_per_s", 0.0), 1),
    }
    if decode_res:
        line["roofline"] = {
            "kernel": "decode_kernel<2,8> (kvattn_decode_partials: split-K partials, "
                      f"{decode_res['n_splits']} splits per KV head)",
            "bound": "hbm",
            "achieved": round(decode_res["kernel_gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(decode_res["kernel_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode"),
            "kernel_us": round(decode_res["kernel_ms"] * 1e3, 2),
            "bytes_per_launch": decode_res["bytes_per_launch"],
            "call_us": round(decode_res["launch_ms"] * 1e3, 2),
            "call_gbs": round(decode_res["launch_gbs"], 2),
        }
    if prefill_res:
        line["prefill"] = {
            "workload": "prefill-262k: 512-token chunk (causal) after 262144 prior tokens, "
                        "2052 pages, 16 layers x 4 KV heads x 24 query heads",
            "tflops": round(prefill_res["tflops"], 2),
            "mfma_frac": round(prefill_res["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "ms_per_step": round(prefill_res["ms_per_step"], 3),
            "tokens_per_s": round(prefill_res["tokens_per_s"], 1),
            "roofline": {
                "kernel": "prefill_kernel (kvattn_prefill_partials: "
                          f"{prefill_res['n_groups']} page groups)",
                "bound": "mfma",
                "achieved": round(prefill_res["kernel_tflops"], 2),
                "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(prefill_res["kernel_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("prefill"),
                "kernel_ms": round(prefill_res["kernel_ms"], 4),
                "call_ms": round(prefill_res["launch_ms"], 4),
            },
        }
        if "cpu_baseline" in prefill_res:
            line["prefill"]["cpu_baseline"] = prefill_res["cpu_baseline"]
        line["prefill"]["gemm_probe"] = gemm_probe(dev)
        log(f"gemm probe: {json.dumps(line['prefill']['gemm_probe'])}")
    if cpu:
        cpu["cpu_model"] = cpu_model()
        cpu["nproc"] = os.cpu_count()
        cpu["one_thread"] = cpu_baseline_tiny_one_thread()
        line["cpu_baseline"] = cpu
    others = {k: v for k, v in extra.items() if k not in (w3.name, synth.WORKLOADS[4].name)}
    if others:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
