"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max-abs <= 2e-2 and mean-abs <= 2e-3 over every compared element, no NaN.
Page slots past kv_len and the pool's trap page are filled with NaN, so any
read of them shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import rpa_workloads as wl
from gpu_common import bitwise_mismatch, compare, gpu_available, make_attn, oracle_rows, run_gpu

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


SMALL = {
    "tiny": lambda: wl.tiny(),
    "decode": lambda: wl.decode(),
    "swa_prefill_1100": lambda: wl.swa_prefill(tokens=1100),
    "global_prefill_777": lambda: wl.global_prefill(tokens=777),
    "mixed_small_w0": lambda: mixed_small(0),
    "mixed_small_w1024": lambda: mixed_small(1024),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name):
    w = SMALL[name]()
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    got = run_gpu(attn, inp)
    ref = oracle_rows(inp)
    mx, mean = compare(got, ref, label=name)
    print(f"{name}: max-abs {mx:.3e} mean-abs {mean:.3e}")


FULL = {
    "swa_prefill": wl.swa_prefill,
    "global_prefill": wl.global_prefill,
    "mixed": lambda: wl.mixed(window=0),
    "mixed_swa": lambda: wl.mixed(window=1024),
    # one GPU's share of the prefills split by KV head (8 and 2 GPUs)
    "swa_prefill_share8": wl.swa_prefill_share8,
    "global_prefill_share2": wl.global_prefill_share2,
}


@pytest.mark.parametrize("name", list(FULL))
def test_parity_full_size_sampled(name):
    """Full-size workloads; the oracle computes a seeded sample of rows one by one."""
    w = FULL[name]()
    print(f"full size {name}", flush=True)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    got = run_gpu(attn, inp)
    t = w.total_q
    cu = inp.cu_q_lens.tolist()
    must = [0, 1, t - 1]
    for s in range(min(w.num_seqs, 4)):
        must += [cu[s], cu[s + 1] - 1, cu[s] + 127, cu[s] + 128, cu[s] + 1023, cu[s] + 1024]
    if w.num_seqs > 4:   # every decode row of the mixed step
        must += list(range(cu[4], t))
    # the first and last token of every query tile the planner made (each
    # token row holds every query head, so every KV head's tile is covered)
    _, items = attn.plan(inp.cu_q_lens, inp.kv_lens, w.window)
    for it in items:
        if it["kind"] == 0:
            must += [it["q_start"], it["q_start"] + it["q_count"] - 1]
    rows = wl.sample_rows(t, 40, w.seed, must)
    ref = oracle_rows(inp, rows)
    mx, mean = compare(got, ref, rows=rows, label=name)
    print(f"{name}: {len(rows)} rows, max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_parity_decode_full_size():
    w = wl.decode()
    inp = wl.make_inputs(w, poison=True)
    got = run_gpu(make_attn(w), inp)
    compare(got, oracle_rows(inp), label="decode")


VARIANTS = [
    ("all_prefill_kernel", {R.RPA_OPT_PATH: 1}),
    ("split32", {R.RPA_OPT_DECODE_SPLIT_KEYS: 32}),
    ("split64", {R.RPA_OPT_DECODE_SPLIT_KEYS: 64}),
    ("split96", {R.RPA_OPT_DECODE_SPLIT_KEYS: 96}),
    ("split_none", {R.RPA_OPT_DECODE_SPLIT_KEYS: 1 << 20}),
    ("decode_rows8", {R.RPA_OPT_DECODE_MAX_ROWS: 8}),
    ("decode_waves8", {R.RPA_OPT_DECODE_WAVES: 8}),
    ("decode_waves4", {R.RPA_OPT_DECODE_WAVES: 4}),
    ("decode_waves4_split32", {R.RPA_OPT_DECODE_WAVES: 4, R.RPA_OPT_DECODE_SPLIT_KEYS: 32}),
    ("decode_waves4_split_none", {R.RPA_OPT_DECODE_WAVES: 4, R.RPA_OPT_DECODE_SPLIT_KEYS: 1 << 20}),
    ("decode_waves8_split32", {R.RPA_OPT_DECODE_WAVES: 8, R.RPA_OPT_DECODE_SPLIT_KEYS: 32}),
    ("decode_waves8_split_none", {R.RPA_OPT_DECODE_WAVES: 8, R.RPA_OPT_DECODE_SPLIT_KEYS: 1 << 20}),
    ("plain_order", {R.RPA_OPT_XCD_GROUPS: 0}),
    ("merge_kernel", {R.RPA_OPT_FUSED_MERGE: 0}),
    ("merge_kernel_split32", {R.RPA_OPT_FUSED_MERGE: 0, R.RPA_OPT_DECODE_SPLIT_KEYS: 32}),
    ("chiplets3", {R.RPA_OPT_XCD_GROUPS: 3}),
    ("single_stream", {R.RPA_OPT_CONCURRENT: 0}),
    ("prefill_split512", {R.RPA_OPT_PREFILL_SPLIT_KEYS: 512}),
    ("prefill_split512_one_stream_merge_kernel", {R.RPA_OPT_PREFILL_SPLIT_KEYS: 512, R.RPA_OPT_CONCURRENT: 0,
                                                  R.RPA_OPT_FUSED_MERGE: 0}),
]


@pytest.mark.parametrize("window", [0, 700])
def test_scheduling_variants_agree(window):
    """Tile/split/merge choices change scheduling, not the result."""
    w = mixed_small(window, seed=300 + window)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    base = run_gpu(make_attn(w), inp)
    compare(base, ref, label="default")
    for label, opts in VARIANTS:
        attn = make_attn(w)
        for k, v in opts.items():
            attn.set_option(k, v)
        got = run_gpu(attn, inp)
        compare(got, ref, label=label)
        d = (got.float() - base.float()).abs().max().item()
        assert d <= 2e-2, f"{label} differs from default by {d}"


def test_multi_token_decode_items_and_splits():
    """q_len 2 with G 8 fits one decode item; splits then hold rows with no visible key."""
    seqs = [(2, 300), (2, 2), (1, 129), (2, 1000), (1, 1)]
    for window in (0, 5, 200):
        w = wl.custom(seqs, 8, 1, 256, 128, window, seed=41)
        inp = wl.make_inputs(w, poison=True)
        ref = oracle_rows(inp)
        for split in (0, 32):
            attn = make_attn(w)
            attn.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, split)
            compare(run_gpu(attn, inp), ref, label=f"w{window}_split{split}")


def test_deterministic_bitwise():
    w = mixed_small(1024, seed=77)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    a = run_gpu(attn, inp).clone()
    b = run_gpu(attn, inp).clone()
    c = run_gpu(make_attn(w), inp)
    for label, other in (("repeated call", b), ("new context", c)):
        bad = bitwise_mismatch(other, a, inp, label)
        assert not bad, bad


@pytest.mark.parametrize("hq,hkv,d,b", [
    (4, 1, 64, 16), (16, 1, 128, 32), (8, 2, 256, 64), (16, 16, 64, 8), (32, 1, 128, 16),
    (16, 2, 512, 128), (8, 8, 512, 256), (2, 1, 256, 1), (12, 4, 128, 128),
    # every page mode at every head size: a tile in one page, a prefill
    # wave's rows in one page, a page per lane; 32- and 16-key decode runs
    (8, 1, 256, 8), (16, 4, 128, 48), (16, 2, 512, 12), (8, 2, 128, 24), (4, 2, 256, 6), (8, 2, 64, 40),
    (16, 2, 512, 6), (8, 2, 64, 128),
])
def test_shapes(hq, hkv, d, b):
    seqs = [(0, 5), (1, 1), (9, 9), (1, 300), (40, 170), (3, 77), (130, 130), (2, 513), (0, 0)]
    for window in (0, 1, 64):
        w = wl.custom(seqs, hq, hkv, d, b, window, seed=hq * 1000 + d + b)
        inp = wl.make_inputs(w, poison=True)
        ref = oracle_rows(inp)
        attn = make_attn(w)
        compare(run_gpu(attn, inp), ref, label=f"hq{hq} hkv{hkv} d{d} b{b} w{window}")


def test_window_one_returns_own_value_exactly():
    w = wl.custom([(7, 20), (1, 300), (50, 50)], 8, 1, 256, 16, 1, seed=3)
    inp = wl.make_inputs(w, poison=True)
    got = run_gpu(make_attn(w), inp).cpu()
    cu, kv = inp.cu_q_lens.tolist(), inp.kv_lens.tolist()
    for s in range(3):
        ql = cu[s + 1] - cu[s]
        for r in range(ql):
            pos = kv[s] - ql + r
            page, slot = int(inp.page_table[s, pos // 16]), pos % 16
            for h in range(8):
                assert torch.equal(got[cu[s] + r, h], inp.v_pages[page, slot, 0])


def test_window_covering_everything_equals_causal():
    w = wl.custom([(100, 300), (1, 200), (64, 64)], 8, 2, 128, 32, 0, seed=5)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    full = run_gpu(attn, inp).clone()
    wide = run_gpu(attn, inp, window=300).clone()
    assert torch.equal(full, wide)


def test_empty_batch_and_empty_sequences():
    w = wl.custom([(0, 10), (0, 0)], 8, 1, 256, 128, 0, seed=6)
    inp = wl.make_inputs(w)
    attn = make_attn(w)
    d = inp.to("cuda")
    out = torch.full((0, 8, 256), 1.0, dtype=torch.bfloat16, device="cuda")
    attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens, 0, 0.1, out=out)
    torch.cuda.synchronize()
    # zero sequences
    attn.forward(d.q, d.k_pages, d.v_pages, d.page_table[:0], [0], [], 0, 0.1, out=out)
    torch.cuda.synchronize()


def test_plan_cache_reuse_and_change():
    """Same metadata reuses the uploaded plan; new metadata replaces it."""
    attn = None
    for seed, seqs in ((1, [(1, 100), (5, 300)]), (2, [(1, 700), (1, 64), (30, 30)]), (1, [(1, 100), (5, 300)])):
        w = wl.custom(seqs, 8, 1, 256, 128, 0, seed=seed, extra_pages_per_seq=8 - (max(k for _, k in seqs) + 127) // 128)
        inp = wl.make_inputs(w, poison=True)
        if attn is None:
            attn = make_attn(w, max_num_seqs=4, max_q_tokens=64)
        for _ in range(2):
            compare(run_gpu(attn, inp), oracle_rows(inp), label=f"seed{seed}")


def test_kernel_timing_leaves_results_unchanged():
    """Timing events only mark the stream: same bits, one duration per launch."""
    w = mixed_small(0, seed=91)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    base = run_gpu(attn, inp).clone()
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 2)
    for _ in range(3):   # the third call is past the cap and is not recorded
        timed = run_gpu(attn, inp)
        assert torch.equal(base, timed)
    info, items = attn.plan(inp.cu_q_lens, inp.kv_lens, w.window)
    prefill_splits = any(it["kind"] == 0 and it["split_group"] >= 0 for it in items)
    for kind, present in ((R.RPA_KERNEL_PREFILL, info["num_prefill_items"] > 0),
                          (R.RPA_KERNEL_DECODE, info["num_decode_items"] > 0),
                          # decode splits merge inside the decode kernel, prefill splits in the merge kernel
                          (R.RPA_KERNEL_MERGE, prefill_splits)):
        t = attn.kernel_times(kind)
        assert len(t) == (2 if present else 0)
        assert np.all(t > 0) and np.all(t < 1000)
        assert len(attn.kernel_times(kind)) == 0   # reading clears the record
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 0)
    assert torch.equal(base, run_gpu(attn, inp))


@pytest.mark.parametrize("window", [0, 300])
def test_fused_merge_matches_merge_kernel_bitwise(window):
    """The last split merges its group with the merge kernel's arithmetic:
    same bits as the separate merge kernel, over repeated calls (the tickets
    must return to zero after every call)."""
    w = wl.custom([(1, int(k)) for k in np.random.default_rng(5).integers(40, 3000, 96)] + [(3, 700), (2, 2)],
                  8, 1, 256, 128, window, seed=17)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    sep = make_attn(w)
    sep.set_option(R.RPA_OPT_FUSED_MERGE, 0)
    sep.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, 64)
    base = run_gpu(sep, inp).clone()
    compare(base, ref, label="merge kernel")
    fused = make_attn(w)
    fused.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, 64)
    info, _ = fused.plan(inp.cu_q_lens, inp.kv_lens, window)
    assert info["num_split_groups"] > 50
    for _ in range(3):
        got = run_gpu(fused, inp)
        assert torch.equal(got, base)
    for d in (64, 512):   # other head sizes, several KV heads
        w2 = wl.custom([(1, 900), (2, 333), (1, 70), (4, 1500)], 16, 4 if d == 64 else 2, d, 64, window, seed=d)
        inp2 = wl.make_inputs(w2, poison=True)
        a = make_attn(w2)
        a.set_option(R.RPA_OPT_DECODE_SPLIT_KEYS, 64)
        compare(run_gpu(a, inp2), oracle_rows(inp2), label=f"fused d{d}")


@pytest.mark.parametrize("hq,hkv,d,b,seqs,window", [
    (8, 2, 128, 64, [(900, 2500), (5, 40), (1, 700), (300, 300)], 0),
    (8, 1, 256, 128, [(600, 2000), (1, 500), (64, 64)], 0),
    (8, 1, 256, 128, [(700, 2100)], 1400),
    (16, 2, 512, 128, [(300, 1800), (2, 9)], 0),
    (4, 1, 64, 16, [(500, 1500), (7, 7)], 0),
    # small pages: one buffer per prefill wave's rows (d 256: 4 rows, d 512: 4 rows)
    (8, 1, 256, 16, [(700, 2100)], 1400),
    (16, 2, 512, 8, [(300, 1800), (2, 9)], 0),
])
def test_prefill_splits(hq, hkv, d, b, seqs, window):
    """Long prefill items cut along their key range: the partial results,
    merged by the merge kernel (several workgroups per group), match the
    oracle, give the same bits whether the decode splits merge in the decode
    kernel or in the merge kernel, and on a repeated call, and agree with the
    unsplit kernel."""
    w = wl.custom(seqs, hq, hkv, d, b, window, seed=d + window)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    fused = make_attn(w)
    fused.set_option(R.RPA_OPT_PREFILL_SPLIT_KEYS, 512)
    info, items = fused.plan(inp.cu_q_lens, inp.kv_lens, window)
    assert info["prefill_split_keys"] == 512
    assert sum(1 for it in items if it["kind"] == 0 and it["split_group"] >= 0) >= 4
    got = run_gpu(fused, inp).clone()
    compare(got, ref, label="prefill splits")
    for _ in range(2):
        assert torch.equal(run_gpu(fused, inp), got)
    sep = make_attn(w)
    sep.set_option(R.RPA_OPT_PREFILL_SPLIT_KEYS, 512)
    sep.set_option(R.RPA_OPT_FUSED_MERGE, 0)
    assert torch.equal(run_gpu(sep, inp), got)
    whole = make_attn(w)
    whole.set_option(R.RPA_OPT_PREFILL_SPLIT_KEYS, -1)
    base = run_gpu(whole, inp)
    compare(base, ref, label="unsplit")
    assert (base.float() - got.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("b", [128, 16, 8, 24, 3])
@pytest.mark.parametrize("window", [0, 333])
def test_prefill_only_calls_head_size_128(b, window):
    """A call with no decode items at head size 128 runs the prefill tile of
    32 keys at three waves per SIMD (8 rows per wave, so page sizes 8 and 16
    read one buffer per wave's rows, 24 and 3 read per lane): oracle parity
    with the key range whole and cut into splits, and the same bits on a
    repeated call.  A decode added to the same call switches back to the
    64-key tile, which must agree with the oracle too."""
    seqs = [(700, 1900), (130, 130), (65, 1000), (33, 97)]
    w = wl.custom(seqs, 8, 2, 128, b, window, seed=b + window)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    for split in (-1, 256):
        attn = make_attn(w)
        attn.set_option(R.RPA_OPT_PREFILL_SPLIT_KEYS, split)
        info, _ = attn.plan(inp.cu_q_lens, inp.kv_lens, window)
        assert info["num_decode_items"] == 0
        got = run_gpu(attn, inp).clone()
        compare(got, ref, label=f"prefill only B={b} W={window} split={split}")
        assert torch.equal(run_gpu(attn, inp), got)
    w2 = wl.custom(seqs + [(1, 500)], 8, 2, 128, b, window, seed=b + window + 1)
    inp2 = wl.make_inputs(w2, poison=True)
    attn = make_attn(w2)
    info, _ = attn.plan(inp2.cu_q_lens, inp2.kv_lens, window)
    assert info["num_decode_items"] > 0
    compare(run_gpu(attn, inp2), oracle_rows(inp2), label=f"with a decode B={b} W={window}")


@pytest.mark.parametrize("n_prefill", [300, 12])
def test_concurrent_decode_stream(n_prefill):
    """Prefill items (more than the compute units, or a few) plus decodes: the
    decode kernel runs on the context's second stream.  Same bits as one
    stream, over repeated calls, and oracle parity."""
    w = wl.custom([(20, 40 + (i % 7)) for i in range(n_prefill)] + [(1, 100 + i) for i in range(60)], 4, 1, 64,
                  16, 0, seed=31)
    inp = wl.make_inputs(w, poison=True)
    ref = oracle_rows(inp)
    one = make_attn(w)
    one.set_option(R.RPA_OPT_CONCURRENT, 0)
    base = run_gpu(one, inp).clone()
    compare(base, ref, label="one stream")
    two = make_attn(w)
    info, _ = two.plan(inp.cu_q_lens, inp.kv_lens, 0)
    assert info["num_prefill_items"] > 0 and info["num_decode_items"] > 0
    for _ in range(3):
        assert torch.equal(run_gpu(two, inp), base)


def test_many_sequences_sampled():
    """A step of 3000 sequences (about 12000 decode items and 400 prefill
    tiles in one call): 2990 decodes of 1-4 tokens over 1-700 keys and ten
    prefill chunks, d 128, G 4, 64-token pages; sampled rows, and a repeated
    call gives the same bits."""
    rng = np.random.default_rng(75)
    seqs = [(int(q), int(q + k)) for q, k in zip(rng.integers(1, 5, 2990), rng.integers(0, 700, 2990))]
    seqs += [(int(q), int(q + k)) for q, k in zip(rng.integers(100, 600, 10), rng.integers(0, 2000, 10))]
    w = wl.custom(seqs, 16, 4, 128, 64, 0, seed=75)
    print(f"many sequences: S={w.num_seqs} T={w.total_q}", flush=True)
    inp = wl.make_inputs(w, poison=True)
    attn = make_attn(w)
    info, _ = attn.plan(inp.cu_q_lens, inp.kv_lens, 0)
    assert info["num_decode_items"] > 2990
    got = run_gpu(attn, inp)
    t = w.total_q
    rows = wl.sample_rows(t, 200, w.seed, [0, 1, t - 1])
    compare(got, oracle_rows(inp, rows), rows=rows, label="many sequences")
    assert torch.equal(run_gpu(attn, inp), got)


def test_long_contexts_sampled():
    """Decodes over 40K-key contexts (many splits per group) and a 2048-token
    chunk on a 30K prefix, with and without a window; sampled rows."""
    seqs = [(1, 40_000), (1, 23_457), (2048, 30_000), (1, 129), (3, 17_001)]
    for window in (0, 1024):
        w = wl.custom(seqs, 8, 1, 256, 128, window, seed=71 + window)
        inp = wl.make_inputs(w, poison=True)
        got = run_gpu(make_attn(w), inp)
        t = w.total_q
        cu = inp.cu_q_lens.tolist()
        must = [0, 1, cu[2], cu[2] + 1, cu[3] - 1, cu[3], t - 1, t - 2, t - 3]
        rows = wl.sample_rows(t, 24, w.seed, must)
        compare(got, oracle_rows(inp, rows), rows=rows, label=f"long w{window}")
