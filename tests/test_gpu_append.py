"""GPU checks of rpa_forward_append (through the C ABI): the step's new K/V
rows are written into their page slots byte for byte as the oracle's append
writes them (every other byte of both pools untouched), and the attention that
follows matches the oracle on the generated pages (max-abs <= 2e-2, mean-abs
<= 2e-3, no NaN).  The new tokens' slots start as NaN, so a row that is not
written, or written to the wrong slot, shows up in the output."""
import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from append_common import stale_pages_and_new_rows
from gpu_common import compare, gpu_available, make_attn, oracle_rows

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def mixed_small(window, seed=205, page_size=128):
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1500, 64)
    chunks = [(300, 300), (150, 230), (70, 400), (33, 80)]
    return wl.Workload(f"mixed_small_w{window}", chunks + [(1, int(k)) for k in kv], 8, 1, 256, page_size,
                       window, seed, length_draw=(64, 1500, 64))


CASES = {
    "tiny": lambda: wl.tiny(),
    "decode": lambda: wl.decode(),
    "decode_pages16": lambda: wl.custom([(1, 64 + 37 * i) for i in range(40)], 8, 1, 256, 16, 0, seed=41),
    "swa_prefill_1100": lambda: wl.swa_prefill(tokens=1100),
    "global_prefill_777": lambda: wl.global_prefill(tokens=777),
    "mixed_small_w0": lambda: mixed_small(0),
    "mixed_small_w1024_pages16": lambda: mixed_small(1024, page_size=16),
    "gqa4_d128_chunks": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 32, 0, seed=42),
    "with_empty_sequences": lambda: wl.custom([(0, 50), (3, 70), (0, 1), (1, 300), (0, 0), (17, 17)], 8, 2, 256, 64,
                                              0, seed=43),
    "mha_d64_window": lambda: wl.custom([(9, 200), (1, 65), (64, 64)], 4, 4, 64, 16, 33, seed=44),
    # page sizes that are not a multiple of 16 keys (a page id per lane in the
    # decode kernel), of 4 (a prefill wave's rows at d 256 in one page), and
    # of 16 but not 32 (16-key decode runs, a prefill wave's rows at d 128)
    "decode_pages8": lambda: wl.custom([(1, 64 + 37 * i) for i in range(40)], 8, 1, 256, 8, 0, seed=46),
    "mixed_small_w1024_pages24": lambda: mixed_small(1024, page_size=24),
    "gqa4_d128_chunks_pages48": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 48, 0,
                                                  seed=49),
    "gqa4_d128_chunks_pages24": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 24, 0,
                                                  seed=50),
}


def run_append(w, attn=None):
    inp = wl.make_inputs(w, poison=True)
    k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp)
    d = inp.to("cuda")
    kp, vp = k_stale.cuda(), v_stale.cuda()
    attn = attn or make_attn(w)
    out = attn.forward_append(d.q, k_new.cuda(), v_new.cuda(), kp, vp, d.page_table, inp.cu_q_lens,
                              inp.kv_lens, w.window, w.scale)
    torch.cuda.synchronize()
    return inp, (k_new, k_stale, v_new, v_stale), kp, vp, out


@pytest.mark.parametrize("name", list(CASES))
def test_append_then_attend(name):
    w = CASES[name]()
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w)
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16)), f"{name}: K pages"
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16)), f"{name}: V pages"
    compare(out, oracle_rows(inp), label=name)


def test_append_matches_forward_on_filled_pages_bitwise():
    """Appending and attending in one call gives the same bits as rpa_forward
    over pages that already hold the rows, on one stream and on two, over
    repeated calls."""
    w = mixed_small(1024)
    inp = wl.make_inputs(w, poison=True)
    d = inp.to("cuda")
    base = make_attn(w).forward(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens,
                                w.window, w.scale).clone()
    for concurrent in (1, 0):
        attn = make_attn(w)
        attn.set_option(R.RPA_OPT_CONCURRENT, concurrent)
        for _ in range(2):
            _, _, kp, vp, out = run_append(w, attn)
            assert torch.equal(out, base), f"concurrent={concurrent}"
            assert torch.equal(kp.cpu().view(torch.int16), inp.k_pages.view(torch.int16))


def test_append_kernel_is_timed():
    """A step whose sequences' tokens span several decode items (every token
    through decode items in chunks) runs the append kernel for them (timed as
    its own kind); a bf16 step of fresh prefills and decodes writes every new
    row in the attention kernels (the prefill kernel its chunks', the decode
    kernel its decodes') and launches none, nor does a step of decodes only."""
    w = mixed_small(0)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_PATH, 3)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    t = attn.kernel_times(R.RPA_KERNEL_APPEND)
    assert len(t) == 1 and t[0] > 0
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    w = wl.custom([(300, 300), (150, 150), (70, 70), (33, 33)] + [(1, 64 + 23 * i) for i in range(64)], 8, 1, 256,
                  128, 0, seed=206)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    assert len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 0
    assert len(attn.kernel_times(R.RPA_KERNEL_PREFILL)) == 1
    assert len(attn.kernel_times(R.RPA_KERNEL_DECODE)) == 1
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    compare(out, oracle_rows(inp), label="fresh prefills and decodes, fused writes")
    w = wl.decode()
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    assert len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 0
    assert len(attn.kernel_times(R.RPA_KERNEL_DECODE)) == 1
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    compare(out, oracle_rows(inp), label="decode, fused write")


@pytest.mark.parametrize("name, seqs, hq, hkv, d, b, window", [
    ("g8_d256_four_tokens", [(4, 200 + 131 * i) for i in range(24)], 8, 1, 256, 128, 700),
    ("g32_d128_pages16", [(1, 64 + 97 * i) for i in range(30)], 32, 1, 128, 16, 0),
    ("g16_d64_two_tokens", [(2, 50 + 61 * i) for i in range(30)], 16, 1, 64, 32, 0),
])
def test_append_in_two_block_decode_items(name, seqs, hq, hkv, d, b, window):
    """The two-block decode kernel (17..32 rows, selected by
    RPA_OPT_DECODE_MAX_ROWS) writes its items' new rows itself as well:
    byte-exact pools, no append kernel, attention within the bar."""
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=81)
    print(f"two-block append {name}", flush=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_DECODE_MAX_ROWS, 32)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    assert len(attn.kernel_times(R.RPA_KERNEL_DECODE2)) == 1
    assert len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 0
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    compare(out, oracle_rows(inp), label=name)


@pytest.mark.parametrize("path", [1, 2])
def test_append_through_one_kernel_kind(path):
    """Every sequence through the prefill kernel (path 1: it writes all
    rows), or decodes wherever their rows fit (path 2)."""
    w = mixed_small(0)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_PATH, path)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    compare(out, oracle_rows(inp), label=f"path {path}")


@pytest.mark.parametrize("name, seqs, hq, hkv, d, b, window, split, fused", [
    # d 256 (32-key tiles, 8 waves of 4 rows): whole tiles in one page (128), each wave's rows in
    # one page (16), a page id per lane (6); chunks without prior context, or whose first new key
    # starts a tile / a wave's run (fused), or sits inside one (the copy kernel writes them)
    ("d256_pages128_fresh", [(150, 150), (300, 300), (70, 70), (1, 90)], 8, 1, 256, 128, 0, 0, True),
    ("d256_pages128_on_tiles", [(150, 214), (33, 65), (300, 300), (70, 390), (1, 90)], 8, 1, 256, 128, 0, 0,
     True),
    ("d256_pages128_inside_tiles", [(150, 230), (33, 80), (70, 400), (1, 90)], 8, 1, 256, 128, 0, 0, False),
    ("d256_pages16_window", [(150, 230), (33, 77), (70, 402), (1, 90)], 8, 1, 256, 16, 100, 0, True),
    ("d256_pages16_inside_runs", [(150, 230), (33, 79), (1, 90)], 8, 1, 256, 16, 100, 0, False),
    ("d256_pages6", [(150, 230), (33, 80), (70, 400), (1, 90)], 8, 1, 256, 6, 0, 0, True),
    # d 128 with a decode (64-key tiles, 16 rows per wave) and without (32-key tiles, 8 rows per wave)
    ("d128_pages48", [(40, 104), (129, 129), (3, 1000), (77, 301)], 16, 4, 128, 48, 0, 0, True),
    ("d128_pages48_inside_runs", [(40, 100), (129, 129), (3, 1000)], 16, 4, 128, 48, 0, 0, False),
    ("d128_pages8_prefill_only", [(40, 104), (129, 129), (77, 301), (5, 37)], 16, 4, 128, 8, 0, 0, True),
    ("d512_pages32", [(45, 333), (16, 16), (1, 50)], 16, 2, 512, 32, 0, 0, True),
    ("d64_pages16_window", [(100, 180), (9, 201), (64, 64)], 8, 2, 64, 16, 33, 0, True),
    ("d64_pages16_inside_runs", [(100, 180), (9, 200), (64, 64)], 8, 2, 64, 16, 33, 0, False),
    # key splits: the first split writes, every split reads the new keys from k_new
    ("d256_splits", [(700, 2108), (1, 500)], 8, 1, 256, 128, 0, 256, True),
    ("d256_splits_pages16", [(700, 2100), (1, 500)], 8, 1, 256, 16, 1400, 256, True),
])
def test_prefill_kernel_writes_the_new_rows(name, seqs, hq, hkv, d, b, window, split, fused):
    """With a bf16 cache the prefill kernel reads a chunk's new keys from
    k_new / v_new and each query tile writes its own tokens' rows, where
    every chunk's first new key starts one of the kernel's buffer runs (a
    tile, or a wave's rows of one; any key with a page id per lane): then no
    append kernel runs (every decode here holds all of its sequence's
    tokens).  Elsewhere the append kernel writes the prefill rows first.
    Either way the pools come out byte for byte as the oracle's append
    leaves them (their new slots start as NaN), the attention matches the
    oracle, and it gives the same bits as rpa_forward over pages that
    already hold the rows."""
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=d + b + window)
    print(f"prefill append {name}", flush=True)

    def configured():
        a = make_attn(w)
        if split:
            a.set_option(R.RPA_OPT_PREFILL_SPLIT_KEYS, split)
        return a

    attn = configured()
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    info, items = attn.plan(inp.cu_q_lens, inp.kv_lens, window)
    assert info["num_prefill_items"] > 0
    if split:
        assert any(it["kind"] == 0 and it["split_index"] > 0 for it in items)
    assert (len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 0) == fused
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16)), f"{name}: K pages"
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16)), f"{name}: V pages"
    compare(out, oracle_rows(inp), label=name)
    dev = inp.to("cuda")
    base = configured().forward(dev.q, dev.k_pages, dev.v_pages, dev.page_table, inp.cu_q_lens, inp.kv_lens,
                                window, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, base), f"{name}: appending call against rpa_forward on filled pages"


def test_long_prefill_launch_keeps_the_copy_kernel():
    """A fresh prefill of more than two prefill workgroups per slot (a
    4608-token causal prefill at d = 512: 576 query tiles) has its rows
    written by the append kernel, which is cheaper there than each
    workgroup's own write: pools byte for byte, sampled rows against the
    oracle."""
    w = wl.global_prefill(tokens=4608)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    info, _ = attn.plan(np.array([0, 4608], np.int32), np.array([4608], np.int32), w.window)
    assert info["num_prefill_items"] > 2 * 256
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    assert len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 1
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    rows = wl.sample_rows(w.total_q, 48, 7, [0, w.total_q - 1])
    compare(out, oracle_rows(inp, rows), rows=rows, label="long prefill, copy kernel")


@pytest.mark.parametrize("fresh", [False, True])
def test_append_in_a_captured_graph(fresh):
    """rpa_forward_append captured into a HIP graph (warm work list) and
    replayed: each replay writes the same rows and gives the eager bits --
    with chunks on prior context (the copy kernel writes their rows) and
    with fresh prefills (the prefill kernel writes them)."""
    w = (wl.custom([(300, 300), (150, 150), (70, 70), (33, 33)] + [(1, 64 + 23 * i) for i in range(64)], 8, 1, 256,
                   128, 1024, seed=207) if fresh else mixed_small(1024))
    inp = wl.make_inputs(w, poison=True)
    k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp)
    d = inp.to("cuda")
    kn, vn = k_new.cuda(), v_new.cuda()
    kp, vp = k_stale.cuda(), v_stale.cuda()
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    eager = attn.forward_append(d.q, kn, vn, kp, vp, d.page_table, inp.cu_q_lens, inp.kv_lens, w.window,
                                w.scale).clone()
    torch.cuda.synchronize()
    assert (len(attn.kernel_times(R.RPA_KERNEL_APPEND)) == 0) == fresh
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 0)
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.forward_append(d.q, kn, vn, kp, vp, d.page_table, inp.cu_q_lens, inp.kv_lens, w.window, w.scale,
                            out=out)
    for _ in range(3):
        kp.copy_(k_stale.cuda())
        vp.copy_(v_stale.cuda())
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(kp.cpu().view(torch.int16), inp.k_pages.view(torch.int16))
        assert torch.equal(vp.cpu().view(torch.int16), inp.v_pages.view(torch.int16))
