"""GPU parity of adaptive host-resident KV streaming (streaming.StreamedDecode):
the newest pages stay on the device and take the appended tokens, the older
history streams from pinned host memory every step, and the LSE merge of the
two equals attention over the whole cache (oracle, decode bar 2e-3). The
resident pool's bytes after the append equal the oracle's quantisation bit for
bit; repeated steps give identical results."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
import long_context_attention_paged_amd as kv
from long_context_attention_paged_amd import streaming
from kvtest_util import DEV, Pools, compare, gpu, host

pytestmark = pytest.mark.gpu

DEC_TOL = 2e-3


@pytest.mark.parametrize("n_kv,gqa,n_q_tok,kv_len,n_hist,n_layers", [
    (2, 6, 4, 40 * 128 - 50, 28, 3),   # verify: history + resident, three layers (both staging slots)
    (1, 6, 1, 9 * 128 + 1, 8, 2),      # decode: the new token opens the resident last page
    (2, 6, 4, 12 * 128, 0, 2),         # no history: everything resident
])
def test_streamed_decode_matches_oracle(n_kv, gqa, n_q_tok, kv_len, n_hist, n_layers):
    g = np.random.default_rng(kv_len + n_hist)
    n_pages = (kv_len + 127) // 128
    n_phys = n_pages + 2
    pos0 = kv_len - n_q_tok
    geom = kv.Geom(n_kv, gqa, n_phys)
    layers, pools, tables, qs, kns, vns = [], [], [], [], [], []
    for _ in range(n_layers):
        table = g.permutation(n_phys)[:n_pages].astype(np.int32)
        p = Pools(n_phys, n_kv, gqa, init_seed=int(g.integers(1 << 30)))
        p.write(g.standard_normal((pos0, n_kv, 256)).astype(np.float32),
                g.standard_normal((pos0, n_kv, 256)).astype(np.float32), 0, table)
        layers.append(streaming.StreamedLayer(geom, p.gk, p.gv, gpu(table, torch.int32), n_pages,
                                              n_hist))
        pools.append(p)
        tables.append(table)
        qs.append(g.standard_normal((n_q_tok, n_kv * gqa, 256)).astype(np.float32))
        kns.append(g.standard_normal((n_q_tok, n_kv, 256)).astype(np.float32))
        vns.append(g.standard_normal((n_q_tok, n_kv, 256)).astype(np.float32))
    sd = streaming.StreamedDecode(geom, layers, n_pages, n_q_tok, DEV)
    q_d, k_d, v_d = [gpu(x) for x in qs], [gpu(x) for x in kns], [gpu(x) for x in vns]
    outs = [torch.empty_like(x) for x in q_d]
    lses = [torch.empty(x.shape[:2], dtype=torch.float32, device=DEV) for x in q_d]
    sd.step(q_d, k_d, v_d, kv_len, 1 / 16, outs, lses)
    torch.cuda.synchronize()
    first = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    sd.step(q_d, k_d, v_d, kv_len, 1 / 16, outs, lses)  # same tokens again: same bytes, same result
    torch.cuda.synchronize()
    for c in range(n_layers):
        assert torch.equal(outs[c], first[c][0]) and torch.equal(lses[c], first[c][1])
        p, table = pools[c], tables[c]
        quant.quantize_into_pool(kns[c], vns[c], pos0, table, p.ok, p.ov)
        L = layers[c]
        rk = host(L.res_k).reshape(L.n_res, n_kv, -1)
        rv = host(L.res_v).reshape(L.n_res, n_kv, -1)
        assert (rk == p.ok[table[n_hist:]]).all() and (rv == p.ov[table[n_hist:]]).all()
        ref_o, ref_l = oracle.decode(qs[c], gqa, p.ok, p.ov, table, n_pages, kv_len, 1 / 16)
        eo, el, rr = compare(outs[c], lses[c], ref_o, ref_l)
        assert eo <= DEC_TOL and el <= 1e-3 and rr <= 2e-3, (c, eo, el, rr)
    assert sd.host_to_device_bytes_per_step() == n_layers * n_hist * n_kv * 53248

