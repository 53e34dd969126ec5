"""GPU checks of stream capture: the attention calls of several layers of one
step (same metadata, each layer its own Q, pages and page table) captured into
one HIP graph and replayed.  Every replay must equal the eager calls bit for
bit, with eager work and synchronisation between the replays; a capture that
would need a new work list is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import rpa_workloads as wl
from gpu_common import bitwise_mismatch, compare, gpu_available, make_attn, oracle_rows

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def mixed_small(window, seed=205):
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1500, 64)
    chunks = [(300, 300), (150, 230), (70, 400), (33, 80)]
    return wl.Workload(f"mixed_small_w{window}", chunks + [(1, int(k)) for k in kv], 8, 1, 256, 128,
                       window, seed, length_draw=(64, 1500, 64))


@pytest.mark.parametrize("window,concurrent", [(1024, 1), (0, 0)])
def test_graph_of_layers_replays_bitwise(window, concurrent):
    w = mixed_small(window)
    layers = 4
    host = [wl.make_inputs(w, seed=w.seed + 7 * i) for i in range(layers)]
    dev = [h.to("cuda") for h in host]
    cu, kv = host[0].cu_q_lens, host[0].kv_lens
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_CONCURRENT, concurrent)
    eager = [attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale).clone()
             for d in dev]
    torch.cuda.synchronize()
    outs = [torch.empty_like(d.q) for d in dev]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d, o in zip(dev, outs):
            attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale, out=o)
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            bad = bitwise_mismatch(o, e, host[i], f"layer {i}")
            assert not bad, bad
    # an eager call after the replays still agrees with the oracle
    rows = wl.sample_rows(w.total_q, 24, w.seed, [0, w.total_q - 1])
    got = attn.forward(dev[2].q, dev[2].k_pages, dev[2].v_pages, dev[2].page_table, cu, kv, w.window, w.scale)
    torch.cuda.synchronize()
    compare(got, oracle_rows(host[2], rows), rows=rows, label="after replays")


def test_capture_with_a_cold_work_list_is_refused():
    w = wl.decode()
    d = wl.make_inputs(w).to("cuda")
    attn = make_attn(w)
    attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, d.cu_q_lens, d.kv_lens, w.window, w.scale)
    torch.cuda.synchronize()
    kv_other = d.kv_lens.clone()
    kv_other[0] += 1            # other metadata: a new work list would be needed
    g = torch.cuda.CUDAGraph()
    with pytest.raises(Exception):
        with torch.cuda.graph(g):
            attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, d.cu_q_lens, kv_other, w.window, w.scale)
    torch.cuda.synchronize()
    # the context still works eagerly afterwards
    out = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, d.cu_q_lens, d.kv_lens, w.window, w.scale)
    torch.cuda.synchronize()
    compare(out, oracle_rows(wl.make_inputs(w)), label="eager after refused capture")
