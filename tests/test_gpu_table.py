"""GPU parity for every entry of the planner's (head size, group, regime,
cache type) table: for each head size d in {64, 128, 256, 512} and group G in
{1, 2, 4, 8, 16, 32}, one call holds a single-token decode, 2- and 4-token
steps, a short chunk and a long prefill, so every regime the table assigns
for that (d, G) runs -- with a bf16 cache the decode kernel (<= 16 rows) and
the prefill kernel; with an fp8 cache also the two-block decode kernel (17..32
rows, d <= 256) and the fp8 prefill route of the head size -- and is compared element by element
with the oracle (page tails and the trap page hold NaN).  The two-block kernel
is also checked on bf16 caches (selected by RPA_OPT_DECODE_MAX_ROWS) with key
splits (fused and separate merge), windows and small pages."""
import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from gpu_common import compare, gpu_available, make_attn, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402

Q_LENS = [1, 2, 4, 9, 300]


def table_kind(d, rows, fp8=False):
    if rows <= 16:
        return 1
    if fp8 and rows <= 32 and d <= 256:
        return 2
    return 0


KIND_TIMING = {0: R.RPA_KERNEL_PREFILL, 1: R.RPA_KERNEL_DECODE, 2: R.RPA_KERNEL_DECODE2}


def table_workload(d, g, seed):
    hkv = 2 if g <= 8 else 1
    return wl.custom([(q, q + 150 + 37 * i) for i, q in enumerate(Q_LENS)], g * hkv, hkv, d, 64, 0, seed=seed)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32])
def test_table_entry_parity(d, g):
    w = table_workload(d, g, 900 + d + g)
    print(f"table bf16 d={d} G={g}", flush=True)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    got = run_gpu(attn, inp)
    compare(got, oracle_rows(inp), label=f"d{d} g{g}")
    kinds = {table_kind(d, q * g) for q in Q_LENS}
    for k, kind in KIND_TIMING.items():
        assert (len(attn.kernel_times(kind)) > 0) == (k in kinds), (d, g, k)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("g", [1, 4, 8, 16, 32])
def test_table_entry_parity_fp8(d, g):
    w = table_workload(d, g, 950 + d + g)
    print(f"table fp8 d={d} G={g}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    base = f.base
    dd = f.to("cuda")
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    out = attn.forward_fp8(dd.base.q, dd.k_pages, dd.v_pages, dd.k_scales, dd.v_scales, dd.base.page_table,
                           base.cu_q_lens, base.kv_lens, 0, base.scale)
    torch.cuda.synchronize()
    ref = ora.forward_fp8_rows(base.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, base.page_table,
                               base.cu_q_lens, base.kv_lens, 0, base.scale)
    compare(out, ref, label=f"fp8 d{d} g{g}")
    kinds = {table_kind(d, q * g, fp8=True) for q in Q_LENS}
    for k, kind in KIND_TIMING.items():
        assert (len(attn.kernel_times(kind)) > 0) == (k in kinds), (d, g, k)
    # the long prefill is always there: staged pages, except at d = 64 and 256,
    # whose E4M3 tiles the prefill kernel converts itself (RPA_OPT_FP8_STAGE's
    # default: two bf16 tiles fit there)
    assert len(attn.kernel_times(R.RPA_KERNEL_STAGE)) == (0 if d in (64, 256) else 1)


TWO_BLOCK = {
    # name: (seqs, Hq, Hkv, d, page_size, window, options)
    "g32_d128_long_splits": ([(1, 64 + 97 * i) for i in range(40)], 32, 1, 128, 128, 0, {}),
    "g32_d128_splits_merge_kernel": ([(1, 64 + 97 * i) for i in range(40)], 32, 1, 128, 128, 0,
                                     {R.RPA_OPT_FUSED_MERGE: 0}),
    "g32_d128_split32": ([(1, 300 + 50 * i) for i in range(12)], 32, 1, 128, 128, 0,
                         {R.RPA_OPT_DECODE_SPLIT_KEYS: 32}),
    "g8_d256_four_tokens_window": ([(4, 200 + 131 * i) for i in range(24)], 8, 1, 256, 128, 700, {}),
    "g16_d64_two_tokens_pages16": ([(2, 50 + 61 * i) for i in range(30)], 16, 1, 64, 16, 0, {}),
    "g32_d256_pages16_window": ([(1, 100 + 83 * i) for i in range(20)], 32, 1, 256, 16, 333, {}),
    "mixed_with_prefill": ([(1, 500), (3, 900), (120, 400), (2, 33), (1, 1)], 8, 1, 256, 128, 0, {}),
}


@pytest.mark.parametrize("name", list(TWO_BLOCK))
def test_two_block_decode_parity(name):
    seqs, hq, hkv, d, b, window, opts = TWO_BLOCK[name]
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=77)
    print(f"two-block {name}", flush=True)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_DECODE_MAX_ROWS, 32)
    for k, v in opts.items():
        attn.set_option(k, v)
    info, items = attn.plan(inp.cu_q_lens, inp.kv_lens, window)
    assert any(it["kind"] == 2 for it in items)
    got = run_gpu(attn, inp)
    ref = oracle_rows(inp)
    compare(got, ref, label=name)
    again = run_gpu(attn, inp)
    assert torch.equal(got, again), "not bitwise reproducible"


@pytest.mark.parametrize("name", ["g32_d128_long_splits", "g8_d256_four_tokens_window"])
def test_two_block_decode_fp8(name):
    seqs, hq, hkv, d, b, window, opts = TWO_BLOCK[name]
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=78)
    f = wl.make_fp8_inputs(w, poison=True)
    base = f.base
    dd = f.to("cuda")
    attn = make_attn(w)
    out = attn.forward_fp8(dd.base.q, dd.k_pages, dd.v_pages, dd.k_scales, dd.v_scales, dd.base.page_table,
                           base.cu_q_lens, base.kv_lens, window, base.scale)
    torch.cuda.synchronize()
    ref = ora.forward_fp8_rows(base.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, base.page_table,
                               base.cu_q_lens, base.kv_lens, window, base.scale)
    compare(out, ref, label=f"fp8 {name}")


def test_two_block_matches_one_block_and_prefill_paths():
    """The same G = 8 four-token step through the prefill kernel (the bf16
    table), through the two-block decode kernel (rows up to 32), through
    16-row decode items of two tokens each (every token in decode items), and
    through the prefill kernel only: all within the oracle's tolerance."""
    w = wl.custom([(4, 100 + 77 * i) for i in range(16)], 8, 1, 256, 128, 0, seed=79)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    for opts in ({}, {R.RPA_OPT_DECODE_MAX_ROWS: 32}, {R.RPA_OPT_PATH: 3}, {R.RPA_OPT_PATH: 1}):
        attn = make_attn(w)
        for k, v in opts.items():
            attn.set_option(k, v)
        compare(run_gpu(attn, inp), ref, label=str(opts))
