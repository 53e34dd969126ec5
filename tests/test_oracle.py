"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: scalar Python loops with ``math.exp`` on tiny inputs;
* a library routine: ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 on CPU after an independent un-paging;
* a hand-worked example with exact rational answers (``tests/golden``);
* closed forms (window 1 returns the own value, constant values, zero keys);
* invariants (rows sum to 1, paging is a pure gather, window >= kv_len is full
  causal, decode equals the last prefill row, a chunk equals the tail of the
  full prefill, GQA equals MHA with repeated KV heads, batch order).

The mutation tests at the bottom plant plausible mistakes *in the oracle* (on
the CPU) and check that at least one pin catches each of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from append_common import new_token_slots, stale_pages_and_new_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers (no oracle code)
# ---------------------------------------------------------------------------

def brute_force(q, kp, vp, pt, cu, kv, window, scale):
    """Scalar loops, straight from the definition, one output element at a time."""
    hq, d = q.shape[1], q.shape[2]
    b, hkv = kp.shape[1], kp.shape[2]
    q = q.to(torch.float64).tolist()
    kp = kp.to(torch.float64).tolist()
    vp = vp.to(torch.float64).tolist()
    pt = pt.tolist()
    cu = [int(x) for x in cu]
    kv = [int(x) for x in kv]
    group = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(cu[-1])]
    for s in range(len(kv)):
        q_len = cu[s + 1] - cu[s]
        for r in range(q_len):
            pos = kv[s] - q_len + r
            for h in range(hq):
                g = h // group
                keys = []
                for j in range(kv[s]):
                    if j > pos:
                        continue
                    if window > 0 and j < pos - window + 1:
                        continue
                    page, slot = pt[s][j // b], j % b
                    dot = 0.0
                    for e in range(d):
                        dot += q[cu[s] + r][h][e] * kp[page][slot][g][e]
                    keys.append((j, scale * dot))
                mx = max(sc for _, sc in keys)
                den = sum(math.exp(sc - mx) for _, sc in keys)
                for e in range(d):
                    acc = 0.0
                    for j, sc in keys:
                        page, slot = pt[s][j // b], j % b
                        acc += math.exp(sc - mx) / den * vp[page][slot][g][e]
                    out[cu[s] + r][h][e] = acc
    return np.array(out, dtype=np.float64).reshape(cu[-1], hq, d)


def sdpa_reference(inp):
    """torch SDPA (float64, CPU) on K/V gathered with flat index arithmetic."""
    q = inp.q.to(torch.float64)
    kp = inp.k_pages.to(torch.float64)
    vp = inp.v_pages.to(torch.float64)
    n_pages, b, hkv, d = kp.shape
    flat_k = kp.reshape(n_pages * b, hkv, d)
    flat_v = vp.reshape(n_pages * b, hkv, d)
    hq = q.shape[1]
    group = hq // hkv
    out = torch.zeros(q.shape, dtype=torch.float64)
    cu = inp.cu_q_lens.tolist()
    kvl = inp.kv_lens.tolist()
    for s in range(len(kvl)):
        q_len, kv_len = cu[s + 1] - cu[s], kvl[s]
        if q_len == 0:
            continue
        t = torch.arange(kv_len)
        idx = inp.page_table[s].long()[t // b] * b + t % b
        k = flat_k[idx].repeat_interleave(group, dim=1).permute(1, 0, 2).contiguous()
        v = flat_v[idx].repeat_interleave(group, dim=1).permute(1, 0, 2).contiguous()
        qs = q[cu[s]:cu[s + 1]].permute(1, 0, 2).contiguous()
        pos = torch.arange(q_len)[:, None] + (kv_len - q_len)
        j = torch.arange(kv_len)[None, :]
        allow = j <= pos
        if inp.window > 0:
            allow = allow & (j > pos - inp.window)
        o = torch.nn.functional.scaled_dot_product_attention(qs, k, v, attn_mask=allow,
                                                             scale=inp.scale)
        out[cu[s]:cu[s + 1]] = o.permute(1, 0, 2)
    return out.numpy()


def run_oracle(inp, window=None, scale=None):
    return ora.forward(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                       inp.kv_lens, inp.window if window is None else window,
                       inp.scale if scale is None else scale)


def small_cases():
    cases = []
    rng = np.random.default_rng(5)
    for hkv in (1, 2, 4):
        for b in (1, 2, 3):
            for window in (0, 1, 2, 3, 100):
                n = int(rng.integers(1, 4))
                seqs = []
                for _ in range(n):
                    kv = int(rng.integers(1, 10))
                    q = int(rng.integers(0, min(kv, 5) + 1))
                    seqs.append((q, kv))
                cases.append(wl.custom(seqs, 4, hkv, 4, b, window, seed=int(rng.integers(1 << 30))))
    return cases


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", small_cases(), ids=lambda w: f"hkv{w.num_kv_heads}_b{w.page_size}_w{w.window}_{len(w.seqs)}seq")
def test_brute_force(w):
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    ref = brute_force(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                      inp.kv_lens, inp.window, inp.scale)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("w", [
    wl.tiny(),
    wl.custom([(5, 40), (0, 7), (33, 33), (1, 90)], 8, 2, 32, 16, 0, seed=11),
    wl.custom([(5, 40), (0, 7), (33, 33), (1, 90)], 8, 2, 32, 16, 17, seed=12),
    wl.custom([(64, 200)], 4, 4, 16, 8, 50, seed=13),
], ids=["tiny", "gqa4_causal", "gqa4_window17", "mha_window50"])
def test_library_sdpa(w):
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    ref = sdpa_reference(inp)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _golden_inputs(fix):
    b, hkv, d = fix["page_size"], fix["num_kv_heads"], fix["head_dim"]
    pt = np.array(fix["page_table"], dtype=np.int64)
    n_pages = int(pt.max()) + 1
    kp = np.full((n_pages, b, hkv, d), np.nan)
    vp = np.full((n_pages, b, hkv, d), np.nan)
    for s, (weights, values) in enumerate(zip(fix["key_weights"], fix["values"])):
        for t, (a, v) in enumerate(zip(weights, values)):
            kp[pt[s][t // b], t % b, 0] = [math.log(a), 0.0]
            vp[pt[s][t // b], t % b, 0] = v
    return (np.array(fix["q"], dtype=np.float64), kp, vp, pt,
            np.array(fix["cu_q_lens"]), np.array(fix["kv_lens"]))


def test_golden_hand_worked():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        fix = json.load(f)
    q, kp, vp, pt, cu, kv = _golden_inputs(fix)
    for window, expect in fix["expected"].items():
        got = ora.forward(q, kp, vp, pt, cu, kv, int(window), fix["scale"])
        want = np.array([[[float(Fraction(x)) for x in row] for row in tok] for tok in expect])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_window_one_returns_own_value():
    w = wl.custom([(7, 20), (1, 5), (3, 3)], 4, 2, 8, 4, 1, seed=3)
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    cu, kv = inp.cu_q_lens.tolist(), inp.kv_lens.tolist()
    vf = inp.v_pages.to(torch.float64).numpy()
    for s in range(len(kv)):
        for r in range(cu[s + 1] - cu[s]):
            pos = kv[s] - (cu[s + 1] - cu[s]) + r
            page, slot = int(inp.page_table[s, pos // 4]), pos % 4
            for h in range(4):
                assert np.array_equal(got[cu[s] + r, h], vf[page, slot, h // 2])


def test_single_token_sequence_returns_v0():
    w = wl.custom([(1, 1)] * 3, 8, 1, 16, 16, 0, seed=4)
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    vf = inp.v_pages.to(torch.float64).numpy()
    for s in range(3):
        page = int(inp.page_table[s, 0])
        for h in range(8):
            assert np.array_equal(got[s, h], vf[page, 0, 0])


@pytest.mark.parametrize("window", [0, 5])
def test_zero_scores_give_mean_of_visible_values(window):
    w = wl.custom([(6, 15), (1, 9)], 4, 1, 8, 4, window, seed=5)
    inp = wl.make_inputs(w, poison=True)
    zero_k = wl.Inputs(w, inp.q, torch.zeros_like(inp.k_pages), inp.v_pages, inp.page_table,
                       inp.cu_q_lens, inp.kv_lens, inp.trap_page, window, inp.scale)
    got_k0 = run_oracle(zero_k)
    got_s0 = run_oracle(inp, scale=0.0)
    cu, kv = inp.cu_q_lens.tolist(), inp.kv_lens.tolist()
    vf = inp.v_pages.to(torch.float64).numpy()
    for s in range(2):
        q_len = cu[s + 1] - cu[s]
        for r in range(q_len):
            pos = kv[s] - q_len + r
            lo = max(0, pos - window + 1) if window else 0
            vals = [vf[int(inp.page_table[s, j // 4]), j % 4, 0] for j in range(lo, pos + 1)]
            mean = np.mean(vals, axis=0)
            for h in range(4):
                np.testing.assert_allclose(got_k0[cu[s] + r, h], mean, rtol=0, atol=1e-13)
                np.testing.assert_allclose(got_s0[cu[s] + r, h], mean, rtol=0, atol=1e-13)


def test_constant_values_give_constant():
    w = wl.custom([(9, 30), (2, 2)], 4, 2, 8, 8, 0, seed=6)
    inp = wl.make_inputs(w)
    v = torch.full_like(inp.v_pages, 0.375)
    c = wl.Inputs(w, inp.q, inp.k_pages, v, inp.page_table, inp.cu_q_lens, inp.kv_lens,
                  inp.trap_page, 0, inp.scale)
    got = run_oracle(c)
    np.testing.assert_allclose(got, 0.375, rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [0, 4])
def test_probability_rows_sum_to_one(window):
    w = wl.custom([(12, 40)], 4, 2, 16, 8, window, seed=7)
    inp = wl.make_inputs(w, poison=True)
    for h in range(4):
        p = ora.sequence_probs(inp.q, inp.k_pages, inp.v_pages, inp.page_table,
                               inp.cu_q_lens, inp.kv_lens, window, inp.scale, 0, h)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        vis = ora.visible(12, 40, window)
        assert np.all(p[~vis] == 0.0)
        assert np.all(p[vis] > 0.0)


def test_paging_is_a_pure_gather():
    """Same logical K/V under a contiguous table, a shuffled table and another page size."""
    w = wl.custom([(10, 37), (1, 12), (20, 20)], 4, 2, 8, 4, 0, seed=8)
    base = wl.make_inputs(w, shuffle=False)
    ref = run_oracle(base)
    rng = np.random.default_rng(1)
    n_pages = base.k_pages.shape[0]
    perm = torch.from_numpy(rng.permutation(n_pages))
    kp = torch.empty_like(base.k_pages)
    vp = torch.empty_like(base.v_pages)
    kp[perm] = base.k_pages
    vp[perm] = base.v_pages
    shuf = wl.Inputs(w, base.q, kp, vp, perm[base.page_table.long()].to(torch.int32),
                     base.cu_q_lens, base.kv_lens, int(perm[base.trap_page]), 0, base.scale)
    assert np.array_equal(run_oracle(shuf), ref)
    # repack into pages of size 3 (contiguous, sequence-major)
    for new_b in (3, 64):
        kv = base.kv_lens.tolist()
        need = [(k + new_b - 1) // new_b for k in kv]
        total = sum(need)
        kp2 = torch.zeros((total + 1, new_b, 2, 8), dtype=torch.bfloat16)
        vp2 = torch.zeros_like(kp2)
        pt2 = torch.full((len(kv), max(need)), total, dtype=torch.int32)
        cur = 0
        for s, k in enumerate(kv):
            for t in range(k):
                src_page, src_slot = int(base.page_table[s, t // 4]), t % 4
                kp2[cur + t // new_b, t % new_b] = base.k_pages[src_page, src_slot]
                vp2[cur + t // new_b, t % new_b] = base.v_pages[src_page, src_slot]
            pt2[s, :need[s]] = torch.arange(cur, cur + need[s])
            cur += need[s]
        re = wl.Inputs(w, base.q, kp2, vp2, pt2, base.cu_q_lens, base.kv_lens, total, 0,
                       base.scale)
        assert np.array_equal(run_oracle(re), ref)


def test_window_covering_everything_is_full_causal():
    w = wl.custom([(10, 37), (1, 12), (20, 20)], 4, 1, 8, 4, 0, seed=9)
    inp = wl.make_inputs(w, poison=True)
    full = run_oracle(inp, window=0)
    for window in (37, 38, 1000):
        assert np.array_equal(run_oracle(inp, window=window), full)
    assert not np.allclose(run_oracle(inp, window=5), full)


def test_decode_equals_last_prefill_row_and_chunk_equals_tail():
    n, prior, chunk = 45, 30, 15
    w_full = wl.custom([(n, n)], 8, 2, 16, 8, 0, seed=10)
    full_in = wl.make_inputs(w_full, shuffle=False)
    full = run_oracle(full_in)
    # decode: one query token (the last one) on the same cache
    dec = wl.Inputs(wl.custom([(1, n)], 8, 2, 16, 8), full_in.q[n - 1:n], full_in.k_pages,
                    full_in.v_pages, full_in.page_table, torch.tensor([0, 1], dtype=torch.int32),
                    full_in.kv_lens, full_in.trap_page, 0, full_in.scale)
    np.testing.assert_allclose(run_oracle(dec)[0], full[n - 1], rtol=0, atol=1e-12)
    # chunk: the last `chunk` tokens with `prior` earlier tokens already cached
    ch = wl.Inputs(wl.custom([(chunk, n)], 8, 2, 16, 8), full_in.q[prior:], full_in.k_pages,
                   full_in.v_pages, full_in.page_table,
                   torch.tensor([0, chunk], dtype=torch.int32), full_in.kv_lens,
                   full_in.trap_page, 0, full_in.scale)
    np.testing.assert_allclose(run_oracle(ch), full[prior:], rtol=0, atol=1e-12)
    # with a window too
    for window in (7,):
        fw = run_oracle(full_in, window=window)
        np.testing.assert_allclose(run_oracle(ch, window=window), fw[prior:], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    w = wl.custom([(9, 21), (1, 14)], 8, 2, 8, 4, 6, seed=11)
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    rep = wl.Inputs(wl.custom(w.seqs, 8, 8, 8, 4, 6), inp.q,
                    inp.k_pages.repeat_interleave(4, dim=2), inp.v_pages.repeat_interleave(4, dim=2),
                    inp.page_table, inp.cu_q_lens, inp.kv_lens, inp.trap_page, 6, inp.scale)
    np.testing.assert_allclose(run_oracle(rep), got, rtol=0, atol=1e-13)


def test_batch_order_permutes_rows_only():
    w = wl.custom([(9, 21), (1, 14), (4, 4), (0, 3)], 4, 1, 8, 4, 0, seed=12)
    inp = wl.make_inputs(w, poison=True)
    got = run_oracle(inp)
    order = [2, 0, 3, 1]
    cu = inp.cu_q_lens.tolist()
    q_parts = [inp.q[cu[s]:cu[s + 1]] for s in order]
    qlens = [cu[s + 1] - cu[s] for s in order]
    cu2 = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    perm_in = wl.Inputs(w, torch.cat(q_parts), inp.k_pages, inp.v_pages,
                        inp.page_table[order], cu2, inp.kv_lens[order], inp.trap_page, 0, inp.scale)
    got2 = run_oracle(perm_in)
    expect = np.concatenate([got[cu[s]:cu[s + 1]] for s in order])
    assert np.array_equal(got2, expect)


def test_row_blocks_and_row_subsets_are_exact(monkeypatch):
    w = wl.custom([(40, 70), (3, 9)], 4, 2, 8, 8, 11, seed=13)
    inp = wl.make_inputs(w, poison=True)
    full = run_oracle(inp)
    monkeypatch.setattr(ora, "ROW_BLOCK", 7)
    np.testing.assert_allclose(run_oracle(inp), full, rtol=0, atol=1e-13)
    rows = [42, 0, 39, 17]
    sub = ora.forward_rows(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                           inp.kv_lens, 11, inp.scale, rows)
    np.testing.assert_allclose(sub, full[rows], rtol=0, atol=1e-13)


def test_metadata_errors():
    w = wl.custom([(2, 4)], 4, 2, 8, 4, 0, seed=14)
    inp = wl.make_inputs(w)
    with pytest.raises(ValueError):
        ora.forward(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                    torch.tensor([1], dtype=torch.int32), 0, 1.0)
    with pytest.raises(ValueError):
        ora.forward(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                    inp.kv_lens, -1, 1.0)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

def _pins_pass() -> bool:
    """Run a compact set of the pins above; False if any of them fails."""
    checks = [
        lambda: test_brute_force(small_cases()[7]),
        lambda: test_brute_force(small_cases()[30]),
        lambda: test_library_sdpa(wl.custom([(5, 40), (0, 7), (33, 33), (1, 90)], 8, 2, 32, 16, 17, seed=12)),
        test_golden_hand_worked,
        test_window_one_returns_own_value,
        test_gqa_equals_mha_with_repeated_kv,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _mut_window_off_by_one(q_len, kv_len, window, rows=None):
    if rows is None:
        rows = np.arange(q_len)
    p = (kv_len - q_len + np.asarray(rows))[:, None]
    j = np.arange(kv_len)[None, :]
    ok = j <= p
    if window > 0:
        ok &= j >= p - window          # W + 1 keys
    return ok


def _mut_query_at_front(q_len, kv_len, window, rows=None):
    if rows is None:
        rows = np.arange(q_len)
    p = np.asarray(rows)[:, None]      # forgets the prior context
    j = np.arange(kv_len)[None, :]
    ok = j <= p
    if window > 0:
        ok &= j >= p - window + 1
    return ok


def _mut_unpage_slot(pages, table_row, kv_len, page_size):
    out = np.empty((kv_len,) + pages.shape[2:], dtype=np.float64)
    for t in range(kv_len):
        out[t] = pages[int(table_row[t // page_size]), (t + 1) % page_size]
    return out


def _mut_softmax_no_normalise(scores, mask):
    s = np.where(mask, scores, -np.inf)
    return np.exp(s - s.max(axis=-1, keepdims=True))


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name,attr,fn", [
    ("window W+1 keys", "visible", _mut_window_off_by_one),
    ("queries placed at the front", "visible", _mut_query_at_front),
    ("wrong page slot", "unpage", _mut_unpage_slot),
    ("softmax not normalised", "softmax_rows", _mut_softmax_no_normalise),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(ora, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"


def test_planted_gqa_mapping_is_caught(monkeypatch):
    real = ora.forward_rows

    def swapped(q, k_pages, v_pages, *a, **k):
        # query head h reads KV head h % Hkv instead of h // G
        qf = ora.as_f64(q)
        hq, hkv = qf.shape[1], k_pages.shape[2]
        g = hq // hkv
        order = [(h % hkv) * g + h // hkv for h in range(hq)]
        inv = np.argsort(order)
        out = real(qf[:, order, :], k_pages, v_pages, *a, **k)
        return out[:, inv, :]
    monkeypatch.setattr(ora, "forward_rows", swapped)
    assert not _pins_pass()


# ---------------------------------------------------------------------------
# KV append (the step's new keys and values into their pages)
# ---------------------------------------------------------------------------

def test_append_golden_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "append_hand_worked.json")))
    shape = (g["num_pages"], g["page_size"], g["num_kv_heads"], g["head_dim"])
    zeros = np.zeros(shape)
    k_out, v_out = ora.append_kv(zeros, zeros, np.array(g["page_table"]), np.array(g["cu_q_lens"]),
                                 np.array(g["kv_lens"]), np.array(g["k_new"], dtype=float),
                                 np.array(g["v_new"], dtype=float))
    want_k, want_v = np.zeros(shape), np.zeros(shape)
    for w in g["expected_written"]:
        want_k[w["page"], w["slot"], 0] = w["k"]
        want_v[w["page"], w["slot"], 0] = w["v"]
    np.testing.assert_array_equal(k_out, want_k)
    np.testing.assert_array_equal(v_out, want_v)
    assert not zeros.any()   # inputs untouched


APPEND_CASES = [
    wl.custom([(5, 40), (0, 7), (33, 33), (1, 90)], 8, 2, 32, 16, 17, seed=12),
    wl.custom([(3, 11), (1, 1), (4, 9)], 4, 4, 8, 3, 0, seed=13),
    wl.custom([(1, 300 + i) for i in range(7)] + [(64, 64)], 8, 1, 16, 128, 0, seed=14),
    wl.custom([(2, 5), (7, 7)], 2, 1, 4, 1, 2, seed=15),
]


@pytest.mark.parametrize("w", APPEND_CASES, ids=lambda w: f"{w.num_seqs}seqs_B{w.page_size}")
def test_append_restores_the_generated_pages(w):
    """Take the new rows out of generated pages (slots set to NaN), append them
    again: every byte of both pools is back as generated."""
    inp = wl.make_inputs(w, poison=True)
    k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp)
    k_out, v_out = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    assert torch.equal(k_out.view(torch.int16), inp.k_pages.view(torch.int16))
    assert torch.equal(v_out.view(torch.int16), inp.v_pages.view(torch.int16))
    assert k_stale.float().isnan().sum() >= len(new_token_slots(inp))   # inputs untouched


@pytest.mark.parametrize("w", APPEND_CASES, ids=lambda w: f"{w.num_seqs}seqs_B{w.page_size}")
def test_append_puts_new_tokens_at_the_last_positions(w):
    """After the append, the un-paged keys and values of every sequence end
    with its new tokens' rows, in order, and attention over the appended pool
    equals attention over the generated one."""
    inp = wl.make_inputs(w)
    k_new, k_stale, v_new, v_stale = stale_pages_and_new_rows(inp, fill=0.0)
    k_out, v_out = ora.append_kv(k_stale, v_stale, inp.page_table, inp.cu_q_lens, inp.kv_lens, k_new, v_new)
    cu, kv, table = inp.cu_q_lens.numpy(), inp.kv_lens.numpy(), inp.page_table.numpy()
    b = inp.k_pages.shape[1]
    for s in range(len(kv)):
        q_len = int(cu[s + 1] - cu[s])
        if q_len == 0:
            continue
        got_k = ora.unpage(ora.as_f64(k_out), table[s], int(kv[s]), b)[-q_len:]
        got_v = ora.unpage(ora.as_f64(v_out), table[s], int(kv[s]), b)[-q_len:]
        np.testing.assert_array_equal(got_k, ora.as_f64(k_new[cu[s]:cu[s + 1]]))
        np.testing.assert_array_equal(got_v, ora.as_f64(v_new[cu[s]:cu[s + 1]]))
    ref = ora.forward_inputs(inp)
    got = ora.forward(inp.q, k_out, v_out, inp.page_table, inp.cu_q_lens, inp.kv_lens, inp.window, inp.scale)
    np.testing.assert_array_equal(got, ref)


def test_planted_append_position_mistake_is_caught(monkeypatch):
    """An append that places token t at position kv_len - q_len + r - 1 (one
    slot early) fails the hand-worked case."""
    def early(k_pages, v_pages, page_table, cu_q_lens, kv_lens, k_new, v_new):
        k_out, v_out = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
        cu, kv, table = ora.as_i64(cu_q_lens), ora.as_i64(kv_lens), ora.as_i64(page_table)
        b = k_pages.shape[1]
        for s in range(len(kv)):
            q_len = int(cu[s + 1] - cu[s])
            for r in range(q_len):
                p = int(kv[s]) - q_len + r - 1
                k_out[int(table[s, p // b]), p % b] = k_new[int(cu[s]) + r]
                v_out[int(table[s, p // b]), p % b] = v_new[int(cu[s]) + r]
        return k_out, v_out
    monkeypatch.setattr(ora, "append_kv", early)
    with pytest.raises(AssertionError):
        test_append_golden_hand_worked()


# ---------------------------------------------------------------------------
# fp8 (OCP E4M3) KV cache with per-KV-head scales
# ---------------------------------------------------------------------------

def _torch_e4m3(codes) -> np.ndarray:
    """torch's own E4M3 decoding (the library routine), as float64."""
    t = codes if isinstance(codes, torch.Tensor) else torch.from_numpy(np.asarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _fp8_pins_pass() -> bool:
    try:
        test_e4m3_matches_torch_for_every_byte()
        test_e4m3_closed_forms()
        test_e4m3_is_monotone_and_symmetric()
        test_fp8_head_scales_fold_into_score_scale_and_output()
    except AssertionError:
        return False
    return True


def test_e4m3_matches_torch_for_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(ora.e4m3_value(codes), _torch_e4m3(codes))


def test_e4m3_closed_forms():
    """Values fixed by the format: bias 7, subnormals m/8 * 2^-6, NaN at 0x7f
    and 0xff, largest finite 448."""
    v = ora.e4m3_value(np.arange(256, dtype=np.uint8))
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
              0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in expect.items():
        assert v[code] == val, hex(code)
    assert math.copysign(1.0, v[0x80]) < 0 and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v[np.r_[0:0x7F, 0x80:0xFF]]).all()


def test_e4m3_is_monotone_and_symmetric():
    v = ora.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.all(np.diff(v[:0x7F]) > 0)
    np.testing.assert_array_equal(v[0x80:0xFF], -v[:0x7F])


def _fp8_case(seqs, hq, hkv, d, b, window, seed):
    w = wl.custom(seqs, hq, hkv, d, b, window=window, seed=seed)
    return wl.make_fp8_inputs(w, poison=True)


def test_fp8_head_scales_fold_into_score_scale_and_output():
    """A K scale c_g multiplies every score of KV head g, so it equals the
    bf16-style forward with scale * c_g; a V scale multiplies that head
    group's output.  The reference side decodes the bytes with torch."""
    f = _fp8_case([(5, 9), (1, 40), (12, 12)], 4, 2, 32, 8, 0, 11)
    b = f.base
    k_val, v_val = _torch_e4m3(f.k_pages), _torch_e4m3(f.v_pages)
    got = ora.forward_fp8_rows(b.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens,
                               b.kv_lens, b.window, b.scale)
    group = 2
    for g in range(2):
        ks, vs = float(f.k_scales[g]), float(f.v_scales[g])
        assert ks != vs
        ref = brute_force(b.q, torch.from_numpy(k_val), torch.from_numpy(v_val), b.page_table, b.cu_q_lens,
                          b.kv_lens, b.window, b.scale * ks)
        heads = slice(g * group, (g + 1) * group)
        np.testing.assert_allclose(got[:, heads], vs * np.asarray(ref)[:, heads], rtol=1e-11, atol=1e-13)


def test_fp8_nan_bytes_past_kv_len_never_contribute():
    f = _fp8_case([(3, 21), (1, 17), (7, 30)], 2, 1, 16, 8, 6, 12)
    b = f.base
    assert (f.k_pages == wl.NAN_E4M3).any()
    got = ora.forward_fp8_rows(b.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens,
                               b.kv_lens, b.window, b.scale)
    assert np.isfinite(got).all()


def test_fp8_pins_pass_on_the_real_oracle():
    assert _fp8_pins_pass()


def _mut_e4m3_no_subnormals(codes):
    c = np.asarray(codes).astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7) / 8.0
    mag = (1.0 + m) * np.exp2(e - 7.0)            # treats exponent 0 as normal
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)



@pytest.mark.parametrize("name", ["no subnormals", "scale of query head", "k and v scales swapped"])
def test_planted_fp8_mistake_is_caught(monkeypatch, name):
    real_dq = ora.dequantize_kv
    if name == "no subnormals":
        monkeypatch.setattr(ora, "e4m3_value", _mut_e4m3_no_subnormals)
    elif name == "scale of query head":
        def dq(pages, scales):   # scale index taken from a wrong (query-head-like) position
            sc = np.asarray(ora.as_f64(scales))[::-1].copy()
            return real_dq(pages, sc)
        monkeypatch.setattr(ora, "dequantize_kv", dq)
    else:
        real_fwd = ora.forward_fp8_rows

        def swapped(q, kp, vp, ks, vs, *a, **k):
            return real_fwd(q, kp, vp, vs, ks, *a, **k)
        monkeypatch.setattr(ora, "forward_fp8_rows", swapped)
    assert not _fp8_pins_pass(), f"planted mistake not caught: {name}"


# ---------------------------------------------------------------------------
# fp8 KV append: the new rows quantized to E4M3 with the per-head scales
# ---------------------------------------------------------------------------

def _e4m3_midpoints():
    v = ora.e4m3_value(np.arange(0x7F))
    return ((v[:-1] + v[1:]) / 2).astype(np.float32)


def test_quantize_e4m3_matches_torch_rounding():
    """torch's float32 -> E4M3 conversion (round to nearest even) on random
    values inside +-448 and on every midpoint between adjacent codes."""
    rng = np.random.default_rng(5)
    mids = _e4m3_midpoints()
    x = np.concatenate([rng.standard_normal(4000) * 40, rng.standard_normal(2000) * 0.02, mids, -mids,
                        [0.0, 1e-30, -1e-30]]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ora.quantize_e4m3(x), want)


def test_quantize_e4m3_closed_forms():
    q = ora.quantize_e4m3
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    np.testing.assert_array_equal(q(ora.e4m3_value(finite).astype(np.float32)), finite)   # every code round-trips
    assert list(q(np.float32([2.0 ** -10, 1.5 * 2.0 ** -10, 3 * 2.0 ** -10]))) == [0x00, 0x01, 0x02]  # ties to even
    assert list(q(np.float32([448.0, 460.0, 1e9, -1e9]))) == [0x7E, 0x7E, 0x7E, 0xFE]                  # saturation
    assert q(np.float32([-0.0]))[0] == 0x80 and q(np.float32([np.nan]))[0] == 0x7F


def test_append_fp8_round_trip_with_power_of_two_scales():
    """New rows that are code value x scale with power-of-two scales divide
    back exactly, so appending them restores the generated bytes."""
    w = wl.custom([(3, 40), (1, 9), (12, 12), (0, 5)], 4, 2, 16, 8, seed=21)
    f = wl.make_fp8_inputs(w)
    b = f.base
    ks = torch.tensor([0.25, 2.0], dtype=torch.float32)
    vs = torch.tensor([0.0625, 1.0], dtype=torch.float32)
    bsz = w.page_size
    slots = [(t, int(fl) // bsz, int(fl) % bsz) for t, fl in enumerate(new_token_slots(b))]
    kval, vval = ora.e4m3_value(f.k_pages.numpy()), ora.e4m3_value(f.v_pages.numpy())
    t_q = b.q.shape[0]
    k_new = np.zeros((t_q, 2, 16)); v_new = np.zeros((t_q, 2, 16))
    for t, page, slot in slots:
        k_new[t] = kval[page, slot] * ks.numpy()[:, None]
        v_new[t] = vval[page, slot] * vs.numpy()[:, None]
    k_stale, v_stale = f.k_pages.clone(), f.v_pages.clone()
    for t, page, slot in slots:
        k_stale[page, slot] = 0x7F
        v_stale[page, slot] = 0x7F
    k_out, v_out = ora.append_kv_fp8(k_stale, v_stale, ks, vs, b.page_table, b.cu_q_lens, b.kv_lens,
                                     torch.from_numpy(k_new).to(torch.bfloat16), torch.from_numpy(v_new).to(torch.bfloat16))
    np.testing.assert_array_equal(k_out, f.k_pages.numpy())
    np.testing.assert_array_equal(v_out, f.v_pages.numpy())


def test_append_fp8_matches_torch_division_and_cast_at_ordinary_scales():
    """A library route for the append's arithmetic at scales that are not
    powers of two: each new element divided by its head's scale in torch's
    float32 (IEEE, correctly rounded) and cast by torch to E4M3 (nearest,
    ties to even) must give the byte the oracle writes into the element's
    slot; every other byte of both pools is left as it was.  The values are
    kept inside +-448 x scale, where torch's cast does not saturate."""
    w = wl.custom([(5, 40), (1, 9), (12, 12), (0, 5), (3, 3)], 6, 3, 32, 8, seed=22)
    f = wl.make_fp8_inputs(w, poison=True)
    b = f.base
    ks = torch.tensor([0.0137, 0.731, 3.3], dtype=torch.float32)
    vs = torch.tensor([0.0291, 1.37, 0.00917], dtype=torch.float32)
    rng = np.random.default_rng(23)
    t_q, hkv, d = b.q.shape[0], 3, 32
    k_new = torch.from_numpy(rng.standard_normal((t_q, hkv, d)).astype(np.float32)) * ks.view(1, -1, 1) * 90
    v_new = torch.from_numpy(rng.standard_normal((t_q, hkv, d)).astype(np.float32)) * vs.view(1, -1, 1) * 90
    k_new = k_new.clamp(-440 * ks.view(1, -1, 1), 440 * ks.view(1, -1, 1)).to(torch.bfloat16)
    v_new = v_new.clamp(-440 * vs.view(1, -1, 1), 440 * vs.view(1, -1, 1)).to(torch.bfloat16)
    k_out, v_out = ora.append_kv_fp8(f.k_pages, f.v_pages, ks, vs, b.page_table, b.cu_q_lens, b.kv_lens, k_new,
                                     v_new)
    want_k, want_v = f.k_pages.clone(), f.v_pages.clone()
    bsz = w.page_size
    for t, fl in enumerate(new_token_slots(b)):
        page, slot = int(fl) // bsz, int(fl) % bsz
        want_k[page, slot] = (k_new[t].to(torch.float32) / ks.view(-1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
        want_v[page, slot] = (v_new[t].to(torch.float32) / vs.view(-1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    np.testing.assert_array_equal(k_out, want_k.numpy())
    np.testing.assert_array_equal(v_out, want_v.numpy())


def test_planted_quantize_ties_away_is_caught(monkeypatch):
    real = ora.quantize_e4m3

    def away(x):
        x = np.asarray(x, dtype=np.float32)
        return real(np.nextafter(x, np.where(x >= 0, np.float32(np.inf), np.float32(-np.inf))))
    monkeypatch.setattr(ora, "quantize_e4m3", away)
    with pytest.raises(AssertionError):
        test_quantize_e4m3_matches_torch_rounding()
