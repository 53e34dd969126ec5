"""GPU checks of what the C ABI promises beyond the arithmetic.

* Keys that no query of a sequence can see (before the window of its first
  query token) are never read into the result, and the page-table entries of
  pages that hold only such keys are never read: the tests fill those slots
  with NaN and point those entries at the NaN trap page, and the result must
  equal the oracle's on the clean inputs (which never look at those keys).
* Work lists are never overwritten while a captured graph may replay them:
  a graph replayed after eager calls with other (larger) metadata, or after
  enough other metadata to evict every uncaptured plan, still gives the eager
  result bit for bit.
* One step of a 5 sliding-window : 1 global layer stack, captured as one graph
  (two work lists: W = 1024 and W = 0), replays bitwise.
* Calls of one context on two streams run in call order.
"""
import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from gpu_common import bitwise_mismatch, compare, gpu_available, make_attn, oracle_rows

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def first_visible_key(q_len: int, kv_len: int, window: int) -> int:
    """The smallest key any query of the sequence may see (0 without a window)."""
    return max(0, kv_len - q_len - window + 1) if window > 0 else 0


def poison_before_window(k_pages, v_pages, page_table, cu, kv, window, page_size, trap, nan_value):
    """Copies of the pools and table with every key before the sequence's first
    visible key set to `nan_value`, and the entries of pages holding only such
    keys pointed at the trap page (input construction only)."""
    k, v, pt = k_pages.clone(), v_pages.clone(), page_table.clone()
    for s in range(len(kv)):
        q_len, kv_len = int(cu[s + 1] - cu[s]), int(kv[s])
        first = first_visible_key(q_len, kv_len, window)
        for t in range(first):
            page = int(page_table[s, t // page_size])
            k[page, t % page_size] = nan_value
            v[page, t % page_size] = nan_value
        for lp in range(first // page_size):
            pt[s, lp] = trap
    return k, v, pt


BEFORE_WINDOW = {
    # name: (seqs, Hq, Hkv, d, page_size, window)
    "d256_b128_prefill_and_decode": ([(300, 300), (150, 700), (1, 500), (7, 900)], 16, 8, 256, 128, 100),
    "d256_b16_first_tile_spans_pages": ([(5, 5), (200, 1313), (1, 333), (40, 97)], 8, 1, 256, 16, 1024),
    "d256_b16_small_window": ([(200, 1313), (1, 333), (70, 700)], 8, 1, 256, 16, 50),
    "d512_b16": ([(90, 600), (1, 400), (33, 80)], 16, 2, 512, 16, 77),
    "d64_b16": ([(120, 500), (1, 170), (64, 64)], 4, 4, 64, 16, 33),
    "d128_b32_g16": ([(5, 400), (1, 300), (60, 260)], 16, 1, 128, 32, 45),
}


@pytest.mark.parametrize("name", list(BEFORE_WINDOW))
def test_keys_before_the_window_are_never_read(name):
    seqs, hq, hkv, d, b, window = BEFORE_WINDOW[name]
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=61)
    print(f"before-window poison {name}", flush=True)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    k, v, pt = poison_before_window(inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens, inp.kv_lens,
                                    window, b, inp.trap_page, float("nan"))
    attn = make_attn(w)
    for path in (0, 1):   # automatic, and every sequence through the prefill kernel
        attn.set_option(R.RPA_OPT_PATH, path)
        out = attn.forward(inp.q.cuda(), k.cuda(), v.cuda(), pt.cuda(), inp.cu_q_lens, inp.kv_lens, window,
                           inp.scale)
        torch.cuda.synchronize()
        compare(out, ref, label=f"{name} path {path}")


@pytest.mark.parametrize("stage", [0, 1])
@pytest.mark.parametrize("name", ["d256_b16_first_tile_spans_pages", "d256_b128_prefill_and_decode", "d512_b16",
                                  "d128_b32_g16", "d64_b16"])
def test_fp8_keys_before_the_window_are_never_read(name, stage):
    """Both fp8 prefill routes: the prefill kernel's E4M3 tile loads clamp to
    the item's key range like the bf16 ones, and the staging route stages
    only pages from the first key its prefill items read (a first tile that
    starts below that key must not look up an unstaged page: the staged
    pool's table holds 0 there)."""
    seqs, hq, hkv, d, b, window = BEFORE_WINDOW[name]
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=62)
    print(f"fp8 before-window poison {name} stage {stage}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    base = f.base
    ref = ora.forward_fp8_rows(base.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, base.page_table,
                               base.cu_q_lens, base.kv_lens, window, base.scale)
    k, v, pt = poison_before_window(f.k_pages, f.v_pages, base.page_table, base.cu_q_lens, base.kv_lens, window,
                                    b, base.trap_page, wl.NAN_E4M3)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = attn.forward_fp8(base.q.cuda(), k.cuda(), v.cuda(), f.k_scales.cuda(), f.v_scales.cuda(), pt.cuda(),
                           base.cu_q_lens, base.kv_lens, window, base.scale)
    torch.cuda.synchronize()
    compare(out, ref, label=f"fp8 {name}")


def small_mixed(window, seed, extra_decodes=0):
    """Three prefill chunks and 48 (+ extra) decodes; page-table rows of 10 pages."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1200, 48 + extra_decodes)
    chunks = [(260, 260), (130, 400), (64, 300)]
    w = wl.Workload(f"small_mixed_w{window}", chunks + [(1, int(k)) for k in kv], 8, 1, 256, 128, window,
                    seed, length_draw=(64, 1200, 48 + extra_decodes))
    w.extra_pages_per_seq = 10 - max(w.pages_needed())
    return w


def test_replay_after_calls_with_larger_metadata_is_bitwise():
    """A captured call keeps its own work list: eager calls with more
    sequences (a larger list that the old code wrote over the captured one)
    and with enough other metadata to evict every uncaptured plan do not
    change what a replay computes."""
    w = small_mixed(1024, seed=401)
    host = wl.make_inputs(w, poison=True)
    d = host.to("cuda")
    cu, kv = host.cu_q_lens, host.kv_lens
    attn = make_attn(w, max_num_seqs=400, max_q_tokens=4096)
    eager = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(d.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale, out=out)
    torch.cuda.synchronize()
    big = small_mixed(0, seed=402, extra_decodes=300)
    bh = wl.make_inputs(big, poison=True)
    bd = bh.to("cuda")
    big_out = attn.forward(bd.q, bd.k_pages, bd.v_pages, bd.page_table, bh.cu_q_lens, bh.kv_lens, 0, big.scale)
    for rep in range(2):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = bitwise_mismatch(out, eager, host, f"replay {rep} after a larger eager call")
        assert not bad, bad
    # twelve more keys: more than the cache keeps, so every uncaptured plan is evicted
    for i in range(12):
        kv_i = bh.kv_lens.clone()
        kv_i[-1] -= i + 1
        attn.forward(bd.q, bd.k_pages, bd.v_pages, bd.page_table, bh.cu_q_lens, kv_i, 0, big.scale)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    bad = bitwise_mismatch(out, eager, host, "replay after evictions")
    assert not bad, bad
    rows = wl.sample_rows(big.total_q, 40, 402, [0, big.total_q - 1])
    compare(big_out, oracle_rows(bh, rows), rows=rows, label="larger eager call")
    # the pinned plan is released; the context keeps working eagerly
    attn.release_captured()
    again = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale)
    torch.cuda.synchronize()
    bad = bitwise_mismatch(again, eager, host, "eager call after the release")
    assert not bad, bad


def test_layer_stack_five_window_one_global_replays_bitwise():
    """One step of a 5:1 stack (five window-1024 layers, then a global one)
    of a mixed chunked-prefill step: six calls, two work lists, one graph."""
    pattern = [1024] * 5 + [0]
    w = small_mixed(1024, seed=403)
    host = [wl.make_inputs(w, seed=w.seed + 11 * i, poison=True) for i in range(len(pattern))]
    dev = [h.to("cuda") for h in host]
    cu, kv = host[0].cu_q_lens, host[0].kv_lens
    attn = make_attn(w)

    def layer_inputs(i):
        return wl.Inputs(w, host[i].q, host[i].k_pages, host[i].v_pages, host[i].page_table, cu, kv,
                         host[i].trap_page, pattern[i], w.scale, True)

    eager = [attn.forward(dd.q, dd.k_pages, dd.v_pages, dd.page_table, cu, kv, win, w.scale).clone()
             for dd, win in zip(dev, pattern)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(dd.q) for dd in dev]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dd, win, o in zip(dev, pattern, outs):
            attn.forward(dd.q, dd.k_pages, dd.v_pages, dd.page_table, cu, kv, win, w.scale, out=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            bad = bitwise_mismatch(o, e, layer_inputs(i), f"replay {rep} layer {i} (W {pattern[i]})")
            assert not bad, bad
    for i in (0, 5):
        compare(eager[i], ora.forward_inputs(layer_inputs(i)), label=f"layer {i} (W {pattern[i]})")


def test_calls_on_two_streams_run_in_call_order():
    """A long prefill call on one stream, then a call with other metadata on a
    second stream right after it: each finds its own work list and the
    library orders the two calls itself."""
    a = wl.swa_prefill(tokens=4096)
    ha = wl.make_inputs(a, poison=True)
    da = ha.to("cuda")
    b = wl.swa_prefill(tokens=1500)
    b.extra_pages_per_seq = a.max_pages_per_seq - b.max_pages_per_seq   # one page-table width
    hb = wl.make_inputs(b, poison=True)
    db = hb.to("cuda")
    attn = make_attn(a)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    out_a = torch.empty_like(da.q)
    out_b = torch.empty_like(db.q)
    with torch.cuda.stream(s1):
        attn.forward(da.q, da.k_pages, da.v_pages, da.page_table, ha.cu_q_lens, ha.kv_lens, a.window, a.scale,
                     out=out_a)
    with torch.cuda.stream(s2):
        attn.forward(db.q, db.k_pages, db.v_pages, db.page_table, hb.cu_q_lens, hb.kv_lens, b.window, b.scale,
                     out=out_b)
    torch.cuda.synchronize()
    rows_a = wl.sample_rows(a.total_q, 32, 5, [0, a.total_q - 1])
    rows_b = wl.sample_rows(b.total_q, 32, 6, [0, b.total_q - 1])
    compare(out_a, oracle_rows(ha, rows_a), rows=rows_a, label="stream 1")
    compare(out_b, oracle_rows(hb, rows_b), rows=rows_b, label="stream 2")


def test_fused_merge_reads_the_splits_writes_not_stale_lines():
    """The split workspace is pooled: a new context's plan takes a block that
    still holds another call's partials.  The last split of a group reads
    its group's partials in the launch that wrote them; a cached line of the
    workspace read earlier in the launch (another group's merge on the same
    compute unit: two slots' LSEs share a 128-byte line) must not stand in
    for them.  Two mixed steps of one shape and different values (their
    decode kernels run beside the prefill kernel, so merges of different
    groups interleave) alternate on fresh contexts, so the one block they
    take holds the other step's partials each time; every result must equal
    the first bit for bit.  (The stale read itself is rare and timing
    dependent: the merges' plain loads gave one wrong decode row in about a
    quarter of the runs of test_replay_after_calls_with_larger_metadata_is_bitwise
    after the append tests, and none in this test's runs.)"""
    wa = wb = small_mixed(1024, seed=401, extra_decodes=150)
    ha, hb = wl.make_inputs(wa, poison=True), wl.make_inputs(wa, seed=1401, poison=True)
    da, db = ha.to("cuda"), hb.to("cuda")

    def fresh_call(w, h, d):
        attn = make_attn(w, max_num_seqs=400, max_q_tokens=4096)
        out = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, h.cu_q_lens, h.kv_lens, w.window, w.scale)
        torch.cuda.synchronize()
        info, _ = attn.plan(h.cu_q_lens, h.kv_lens, w.window)
        attn.close()
        return out, info

    first, info = fresh_call(wa, ha, da)
    assert info["num_split_groups"] >= 100
    rows = wl.sample_rows(wa.total_q, 48, 501, [0, wa.total_q - 1] + list(range(454, wa.total_q)))
    compare(first, oracle_rows(ha, rows), rows=rows, label="first call")
    for i in range(16):
        fresh_call(wb, hb, db)
        again, _ = fresh_call(wa, ha, da)
        bad = bitwise_mismatch(again, first, ha, f"call {i + 2} after the other step")
        assert not bad, bad


@pytest.mark.parametrize("page_size", [128, 16, 8])
@pytest.mark.parametrize("mode", ["bf16", "bf16_append", "fp8_staged", "fp8_converting"])
def test_pages_past_4gib_give_the_same_bits(mode, page_size):
    """Every page address is 64-bit: the same pages placed past the first
    4 GiB of a pool of more than 4 GiB per tensor (page-table entries moved
    up by as many pages) give bit for bit the result of a small pool, in
    every page mode (a page per tile or chunk, per run of 16 keys or of a
    wave's rows, per lane) and with an fp8 cache both ways; an appending
    call writes the same bytes there."""
    from append_common import stale_pages_and_new_rows
    w = wl.custom([(60, 300), (1, 517), (1, 90), (200, 200), (3, 1000), (1, 33)], 8, 2, 128, page_size, 0,
                  seed=600 + page_size)
    fp8 = mode.startswith("fp8")
    if fp8:
        f = wl.make_fp8_inputs(w, poison=True)
        inp, k_small, v_small = f.base, f.k_pages, f.v_pages
    else:
        inp = wl.make_inputs(w, poison=True)
        k_small, v_small = inp.k_pages, inp.v_pages
    if mode == "bf16_append":
        k_new, k_small, v_new, v_small = stale_pages_and_new_rows(inp)
    page_bytes = k_small[0].numel() * k_small.element_size()
    base = -(-(int(4.25 * 2 ** 30)) // page_bytes)   # first page id past 4.25 GiB
    n_pages = k_small.shape[0]

    def run(k, v, table):
        attn = make_attn(w)
        if fp8:
            attn.set_option(R.RPA_OPT_FP8_STAGE, 1 if mode == "fp8_staged" else 0)
            out = attn.forward_fp8(inp.q.cuda(), k, v, f.k_scales.cuda(), f.v_scales.cuda(), table, inp.cu_q_lens,
                                   inp.kv_lens, 0, w.scale)
        elif mode == "bf16_append":
            out = attn.forward_append(inp.q.cuda(), k_new.cuda(), v_new.cuda(), k, v, table, inp.cu_q_lens,
                                      inp.kv_lens, 0, w.scale)
        else:
            out = attn.forward(inp.q.cuda(), k, v, table, inp.cu_q_lens, inp.kv_lens, 0, w.scale)
        torch.cuda.synchronize()
        attn.close()
        return out

    ks, vs = k_small.cuda(), v_small.cuda()
    small = run(ks, vs, inp.page_table.cuda()).clone()
    kb = torch.zeros((base + n_pages,) + tuple(k_small.shape[1:]), dtype=k_small.dtype, device="cuda")
    vb = torch.zeros_like(kb)
    kb[base:] = k_small.cuda()
    vb[base:] = v_small.cuda()
    big = run(kb, vb, (inp.page_table + base).cuda())
    assert kb.numel() * kb.element_size() > 4 * 2 ** 30
    bad = bitwise_mismatch(big, small, inp, f"{mode} B{page_size}: pages past 4 GiB")
    assert not bad, bad
    if mode == "bf16_append":
        assert torch.equal(kb[base:].view(torch.int16), ks.view(torch.int16))
        assert torch.equal(vb[base:].view(torch.int16), vs.view(torch.int16))
    del kb, vb
    torch.cuda.empty_cache()
