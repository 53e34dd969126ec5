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
    """A mixed step runs the append kernel for its prefill chunks (timed as its
    own kind); a step of decodes only writes every new row in the decode
    kernel (the fused write) and launches no append kernel."""
    w = mixed_small(0)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    run_append(w, attn)
    t = attn.kernel_times(R.RPA_KERNEL_APPEND)
    assert len(t) == 1 and t[0] > 0
    assert len(attn.kernel_times(R.RPA_KERNEL_DECODE)) == 1
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
    """Every sequence through the prefill kernel (path 1: the append kernel
    writes all rows), or decodes wherever their rows fit (path 2)."""
    w = mixed_small(0)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_PATH, path)
    inp, (k_new, k_stale, v_new, v_stale), kp, vp, out = run_append(w, attn)
    want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
    compare(out, oracle_rows(inp), label=f"path {path}")


def test_append_in_a_captured_graph():
    """rpa_forward_append captured into a HIP graph (warm work list) and
    replayed: each replay writes the same rows and gives the eager bits."""
    w = mixed_small(1024)
    inp = wl.make_inputs(w, poison=True)
    k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp)
    d = inp.to("cuda")
    kn, vn = k_new.cuda(), v_new.cuda()
    kp, vp = k_stale.cuda(), v_stale.cuda()
    attn = make_attn(w)
    eager = attn.forward_append(d.q, kn, vn, kp, vp, d.page_table, inp.cu_q_lens, inp.kv_lens, w.window,
                                w.scale).clone()
    torch.cuda.synchronize()
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
