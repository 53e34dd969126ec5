"""GPU parity over seeded random calls (through the C ABI).

Each case draws a head size, head counts, page size, a ragged batch (single
token decodes, short chunks, whole prefills and chunks on prior context of
up to 900 keys), a window and every scheduling option of the library
(paths, split sizes, waves, the fused or separate merge, the second stream,
the fp8 prefill route), then checks every element of the call against the
oracle: a bf16 cache through rpa_forward or rpa_forward_append (whose pools
must also come out bit for bit as the oracle's append leaves them), or an
fp8 cache through rpa_forward_fp8 or rpa_forward_fp8_append (pools byte for
byte as the oracle's fp8 append).  Page slots past kv_len and the trap page
hold NaN, so a read of them shows in the output.  The options change only
the schedule, so every draw has the same bar: max-abs <= 2e-2, mean-abs <=
2e-3, no NaN.  RPA_RANDOM_CALLS=<n> draws n calls instead of 48.

Larger calls (up to 48 sequences of up to 5000 keys: long prefill splits,
many decode splits; no fp8 append, whose oracle quantizes element by
element) are drawn the same way and checked on sampled token rows: every
row of a sequence of at most 4 tokens, and 96 others with each sequence's
first and last (RPA_RANDOM_LARGE_CALLS=<n>, default 12).
"""
import os

import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from append_common import new_token_slots, stale_pages_and_new_rows
from gpu_common import compare, gpu_available, make_attn, oracle_rows

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402

HEADS = [(1, 1), (2, 1), (4, 1), (8, 1), (16, 1), (32, 1), (4, 2), (8, 2), (16, 4), (4, 4), (8, 8)]
PAGE_SIZES = [1, 3, 8, 16, 24, 32, 48, 64, 128]
MAX_ROWS = 4096   # query tokens x query heads per call, so the oracle takes seconds


def draw(seed, large=False):
    """(workload, options, mode) of one random call."""
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256, 512]))
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    b = int(rng.choice(PAGE_SIZES if not large else PAGE_SIZES[2:]))
    seqs = []
    for _ in range(int(rng.integers(1, 9 if not large else 49))):
        kv = int(rng.integers(1, 901 if not large else 5001))
        kind = int(rng.integers(5))
        q = [1, int(rng.integers(1, min(kv, 40) + 1)), kv, int(rng.integers(0, kv + 1)), 0][kind]
        seqs.append([min(q, kv), kv])
    if large:
        # pools of at most 2^26 elements each: drop the longest sequences
        while len(seqs) > 1 and sum(k for _, k in seqs) * hkv * d > (1 << 26):
            seqs.pop(int(np.argmax([k for _, k in seqs])))
    else:
        # keep the oracle's work small: shorten the query spans, longest first
        while sum(q for q, _ in seqs) * hq > MAX_ROWS:
            i = int(np.argmax([q for q, _ in seqs]))
            seqs[i][0] //= 2
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 1001))
    opts = {
        R.RPA_OPT_PATH: int(rng.choice([0, 0, 0, 1, 2, 3])),
        R.RPA_OPT_DECODE_SPLIT_KEYS: int(rng.choice([0, 0, 32, 64, 160, 512])),
        R.RPA_OPT_DECODE_MAX_ROWS: int(rng.choice([0, 0, 16, 32])),
        R.RPA_OPT_DECODE_WAVES: int(rng.choice([0, 4, 8])),
        R.RPA_OPT_FUSED_MERGE: int(rng.choice([1, 1, 0])),
        R.RPA_OPT_PREFILL_SPLIT_KEYS: int(rng.choice([0, 0, -1, 512, 1024])),
        R.RPA_OPT_CONCURRENT: int(rng.choice([1, 1, 0])),
        R.RPA_OPT_XCD_GROUPS: int(rng.choice([8, 8, 1, 3])),
        R.RPA_OPT_FP8_STAGE: int(rng.choice([2, 0, 1])),
    }
    # (the oracle's fp8 quantizer is a scalar loop: large calls leave the fp8 append out)
    mode = str(rng.choice(["forward", "forward", "append", "fp8"] + ([] if large else ["fp8_append"])))
    w = wl.custom([tuple(x) for x in seqs], hq, hkv, d, b, window, seed=seed,
                  extra_pages_per_seq=int(rng.integers(0, 3)), name=f"random_{seed}")
    return w, opts, mode


def configured(w, opts):
    attn = make_attn(w)
    for k, v in opts.items():
        attn.set_option(k, v)
    return attn


def checked_rows(w, large):
    """Token rows compared with the oracle: all, or for a large call every row
    of sequences of at most 4 tokens plus a seeded sample with every
    sequence's first and last row."""
    if not large:
        return None
    cu = np.concatenate([[0], np.cumsum([q for q, _ in w.seqs])])
    must = [int(x) for s in range(len(w.seqs)) if cu[s + 1] > cu[s]
            for x in ((range(cu[s], cu[s + 1]) if cu[s + 1] - cu[s] <= 4 else (cu[s], cu[s + 1] - 1)))]
    return wl.sample_rows(int(cu[-1]), 96, w.seed, must)


def run_random(seed, large):
    w, opts, mode = draw(seed, large)
    print(f"random call {seed}: {mode} d={w.head_dim} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"B={w.page_size} W={w.window} seqs={w.seqs} opts={opts}", flush=True)
    attn = configured(w, opts)
    rows = checked_rows(w, large)
    if mode in ("fp8", "fp8_append"):
        f = wl.make_fp8_inputs(w, poison=True)
        b = f.base
        d = b.to("cuda")
        kp, vp = f.k_pages, f.v_pages
        if mode == "fp8":
            out = attn.forward_fp8(d.q, kp.cuda(), vp.cuda(), f.k_scales.cuda(), f.v_scales.cuda(), d.page_table,
                                   b.cu_q_lens, b.kv_lens, b.window, b.scale)
        else:
            flat = torch.from_numpy(new_token_slots(b))
            hd = (w.num_kv_heads, w.head_dim)
            k_new = b.k_pages.reshape(-1, *hd)[flat].contiguous()
            v_new = b.v_pages.reshape(-1, *hd)[flat].contiguous()
            k_stale, v_stale = f.k_pages.clone(), f.v_pages.clone()
            k_stale.reshape(-1, *hd)[flat] = wl.NAN_E4M3
            v_stale.reshape(-1, *hd)[flat] = wl.NAN_E4M3
            kp, vp = ora.append_kv_fp8(k_stale, v_stale, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens,
                                       b.kv_lens, k_new, v_new)
            kd, vd = k_stale.cuda(), v_stale.cuda()
            out = attn.forward_fp8_append(d.q, k_new.cuda(), v_new.cuda(), kd, vd, f.k_scales.cuda(),
                                          f.v_scales.cuda(), d.page_table, b.cu_q_lens, b.kv_lens, b.window, b.scale)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(kd.cpu().numpy(), np.asarray(kp))
            np.testing.assert_array_equal(vd.cpu().numpy(), np.asarray(vp))
        torch.cuda.synchronize()
        ref = ora.forward_fp8_rows(b.q, kp, vp, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens, b.kv_lens,
                                   b.window, b.scale, rows)
        compare(out, ref, rows=rows, label=f"random {seed} {mode}")
        return
    inp = wl.make_inputs(w, poison=True)
    d = inp.to("cuda")
    if mode == "append":
        k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp)
        kp, vp = k_stale.cuda(), v_stale.cuda()
        out = attn.forward_append(d.q, k_new.cuda(), v_new.cuda(), kp, vp, d.page_table, inp.cu_q_lens,
                                  inp.kv_lens, w.window, w.scale)
        torch.cuda.synchronize()
        want_k, want_v = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
        assert torch.equal(kp.cpu().view(torch.int16), torch.as_tensor(want_k).view(torch.int16)), "K pages"
        assert torch.equal(vp.cpu().view(torch.int16), torch.as_tensor(want_v).view(torch.int16)), "V pages"
    else:
        out = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens, w.window,
                           w.scale)
        torch.cuda.synchronize()
    compare(out, oracle_rows(inp, rows), rows=rows, label=f"random {seed} {mode}")


@pytest.mark.parametrize("seed", range(9000, 9000 + int(os.environ.get("RPA_RANDOM_CALLS", "48"))))
def test_random_call(seed):
    run_random(seed, large=False)


@pytest.mark.parametrize("seed", range(7000, 7000 + int(os.environ.get("RPA_RANDOM_LARGE_CALLS", "12"))))
def test_random_large_call(seed):
    run_random(seed, large=True)
