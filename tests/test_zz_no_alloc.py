"""GPU checks of rpa_forward_noalloc (through the C ABI): the entry point that
allocates nothing, with its work list and split partials in the library's
static scratch array, gives the same result as rpa_forward -- bit for bit, and
within the oracle's tolerance -- on two calls in a row, the second with a
smaller input; a call whose list and partials exceed the scratch is refused
with an error before anything is launched."""
import numpy as np
import pytest
import torch

import rpa_workloads as wl
from gpu_common import compare, gpu_available, make_attn, oracle_rows

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def mixed_small(window, seed, decodes):
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1500, decodes)
    chunks = [(300, 300), (150, 230), (70, 400), (33, 80)]
    w = wl.Workload(f"mixed_small_w{window}", chunks + [(1, int(k)) for k in kv], 8, 1, 256, 128, window, seed,
                    length_draw=(64, 1500, decodes))
    w.extra_pages_per_seq = 12 - max(w.pages_needed())
    return w


def run_both(attn, inp):
    d = inp.to("cuda")
    ref = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens, inp.window, inp.scale)
    out = torch.full_like(d.q, float("nan"))
    attn.forward_noalloc(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens, inp.window, inp.scale,
                         out=out)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("window,opts", [(0, {}), (1024, {}),
                                         (0, {R.RPA_OPT_PREFILL_SPLIT_KEYS: 256, R.RPA_OPT_CONCURRENT: 0})],
                         ids=["causal", "window1024", "prefill_splits"])
def test_noalloc_matches_rpa_forward_on_two_calls(window, opts):
    big = mixed_small(window, seed=501, decodes=64)
    small = mixed_small(window, seed=502, decodes=20)
    attn = make_attn(big)
    for k, v in opts.items():
        attn.set_option(k, v)
    for label, w in (("first call", big), ("second, smaller call", small)):
        print(f"noalloc {label} W={window} opts={opts}: seqs={w.num_seqs} T={w.total_q}", flush=True)
        inp = wl.make_inputs(w, poison=True)
        out, ref = run_both(attn, inp)
        assert torch.equal(out, ref), f"{label}: differs from rpa_forward"
        compare(out, oracle_rows(inp), label=label)
    info = attn.plan_info(wl.make_inputs(big).cu_q_lens, wl.make_inputs(big).kv_lens, window)
    assert info["num_split_groups"] > 0   # the merge kernel ran on scratch partials


def test_noalloc_decode_batch_and_prefill_alternate():
    """The decode batch, then an 8192-token window prefill (no partials), then
    the decode batch again: each equals rpa_forward bit for bit."""
    dec = wl.decode()
    pre = wl.swa_prefill(tokens=2048, num_q_heads=8, num_kv_heads=1)
    pre.extra_pages_per_seq = max(0, dec.max_pages_per_seq - pre.max_pages_per_seq)
    dec.extra_pages_per_seq = max(0, pre.max_pages_per_seq - dec.max_pages_per_seq)
    attn = make_attn(dec, max_num_seqs=dec.num_seqs, max_q_tokens=2048)
    for w in (dec, pre, dec):
        print(f"noalloc {w.name}", flush=True)
        inp = wl.make_inputs(w, poison=True)
        out, ref = run_both(attn, inp)
        assert torch.equal(out, ref), w.name


def test_noalloc_refuses_a_call_beyond_the_scratch():
    """d = 512 decodes cut into 32-key splits need more partial slots than the
    scratch holds: the call fails with a message and launches nothing (the
    output keeps its fill); a later call that fits still works."""
    w = wl.custom([(1, 600 + 7 * i) for i in range(128)], 8, 1, 512, 128, 0, seed=503)
    inp = wl.make_inputs(w, poison=True)
    d = inp.to("cuda")
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, 32)
    out = torch.full_like(d.q, 7.0)
    with pytest.raises(R.RpaError) as e:
        attn.forward_noalloc(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens, 0, inp.scale,
                             out=out)
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    attn.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, 0)
    got, ref = run_both(attn, inp)
    assert torch.equal(got, ref)
