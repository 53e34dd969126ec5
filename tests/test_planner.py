"""Host planner (work-list builder) properties, through rpa_plan on the CPU.

Every (token, query head) must be covered by exactly one item or one split
group, whose key ranges are exactly the keys that token can see (checked
against the oracle's visibility rule by brute force); splits partition their
group's range; lists are deterministic and longest-first.
"""
import numpy as np
import pytest

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from ragged_paged_attention_forward_amd import (RPA_OPT_DECODE_MAX_ROWS, RPA_OPT_DECODE_SPLIT_KEYS,
                                                RPA_OPT_PATH, RPA_OPT_PREFILL_SPLIT_KEYS, RPA_OPT_XCD_GROUPS,
                                                RaggedPagedAttention, metrics)


def plan_for(w, options=()):
    attn = RaggedPagedAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                max(1, w.num_seqs), w.max_pages_per_seq, max(1, w.total_q))
    for k, v in options:
        attn.set_option(k, v)
    cu = np.concatenate([[0], np.cumsum([q for q, _ in w.seqs])]).astype(np.int32)
    kv = np.array([k for _, k in w.seqs], dtype=np.int32)
    info, items = attn.plan(cu, kv, w.window)
    attn.close()
    return cu, kv, info, items


def check_plan(w, cu, kv, info, items):
    g_ratio = w.num_q_heads // w.num_kv_heads
    assert info["num_prefill_items"] + info["num_decode_items"] == len(items)
    assert info["visible_pairs"] == metrics.visible_pairs(w.seqs, w.window)
    cover = {}   # (token, kv_head) -> list of items
    for it in items:
        s, g = it["seq"], it["kv_head"]
        assert 0 <= g < w.num_kv_heads
        assert cu[s] <= it["q_start"] and it["q_start"] + it["q_count"] <= cu[s + 1]
        assert it["q_count"] >= 1
        assert 0 <= it["kv_begin"] < it["kv_end"] <= kv[s]
        assert it["q_pos0"] == kv[s] - (cu[s + 1] - cu[s]) + (it["q_start"] - cu[s])
        if it["kind"] == 1:
            assert it["q_count"] * g_ratio <= 16
        elif it["kind"] == 2:
            assert 16 < it["q_count"] * g_ratio <= 32 and w.head_dim <= 256
        else:
            assert it["kind"] == 0
            assert it["q_count"] * g_ratio <= info["prefill_rows"]
        for t in range(it["q_start"], it["q_start"] + it["q_count"]):
            cover.setdefault((t, g), []).append(it)
    for s in range(len(kv)):
        q_len = cu[s + 1] - cu[s]
        vis = ora.visible(q_len, kv[s], w.window)
        for r in range(q_len):
            want = set(np.nonzero(vis[r])[0].tolist())
            for g in range(w.num_kv_heads):
                its = cover[(cu[s] + r, g)]
                groups = {it["split_group"] for it in its}
                assert len(groups) == 1
                if groups == {-1}:
                    assert len(its) == 1
                else:
                    n = its[0]["num_splits"]
                    assert len(its) == n
                    assert sorted(it["split_index"] for it in its) == list(range(n))
                    assert len({it["partial_base"] for it in its}) == 1
                    assert len({it["kind"] for it in its}) == 1
                    if its[0]["kind"] == 0:   # prefill splits meet on 64-key boundaries
                        cuts = sorted(it["kv_begin"] for it in its)[1:]
                        assert all(c % 64 == 0 for c in cuts)
                # union of the item key ranges, no overlap between splits
                keys = []
                for it in sorted(its, key=lambda x: x["kv_begin"]):
                    keys.extend(range(it["kv_begin"], it["kv_end"]))
                assert len(keys) == len(set(keys))
                keys = set(keys)
                assert want <= keys
                # tight: the item range is the union over the item's rows
                lo = min(it["kv_begin"] for it in its)
                hi = max(it["kv_end"] for it in its)
                rows = range(its[0]["q_start"] - cu[s], its[0]["q_start"] - cu[s] + its[0]["q_count"])
                union = np.nonzero(vis[list(rows)].any(axis=0))[0]
                assert lo == union.min() and hi == union.max() + 1
    # partial-result slots: each group owns num_splits blocks of 16 rows (decode) or
    # of prefill_rows rows (prefill), disjoint and within num_partials
    used = []
    for grp in {(it["split_group"], it["partial_base"], it["num_splits"], it["kind"])
                for it in items if it["split_group"] >= 0}:
        per = {1: 1, 2: 2}.get(grp[3], info["prefill_rows"] // 16)
        used.extend(range(grp[1], grp[1] + grp[2] * per))
    assert len(used) == len(set(used))
    assert all(0 <= u < info["num_partials"] for u in used)


WORKLOADS = [
    wl.tiny(), wl.decode(), wl.swa_prefill(tokens=700), wl.global_prefill(tokens=300),
    wl.custom([(2, 300), (2, 2), (1, 129), (2, 1000), (1, 1), (0, 5), (40, 170)], 8, 1, 256, 128, 0, 1),
    wl.custom([(2, 300), (2, 2), (1, 129), (2, 1000), (1, 1), (0, 5), (40, 170)], 8, 1, 256, 128, 100, 1),
    wl.custom([(5, 77), (1, 1), (130, 130), (3, 513)], 16, 1, 128, 16, 64, 2),
    wl.custom([(5, 77), (1, 1), (130, 130), (3, 513)], 32, 1, 128, 16, 0, 3),
    wl.custom([(9, 9), (1, 300)], 12, 4, 64, 1, 1, 4),
]


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name + f"_w{w.window}_g{w.num_q_heads // w.num_kv_heads}")
def test_plan_covers_exactly_the_visible_keys(w):
    cu, kv, info, items = plan_for(w)
    check_plan(w, cu, kv, info, items)


@pytest.mark.parametrize("options", [
    [(RPA_OPT_PATH, 1)], [(RPA_OPT_PATH, 2)], [(RPA_OPT_DECODE_SPLIT_KEYS, 32)],
    [(RPA_OPT_DECODE_SPLIT_KEYS, 100)], [(RPA_OPT_DECODE_SPLIT_KEYS, 1 << 20)],
    [(RPA_OPT_DECODE_MAX_ROWS, 8)], [(RPA_OPT_DECODE_MAX_ROWS, 1)],
])
def test_plan_options_keep_coverage(options):
    w = WORKLOADS[5]
    cu, kv, info, items = plan_for(w, options)
    check_plan(w, cu, kv, info, items)
    opts = dict(options)
    if opts.get(RPA_OPT_PATH) == 1:
        assert info["num_decode_items"] == 0
    if RPA_OPT_DECODE_SPLIT_KEYS in opts:
        split = -(-opts[RPA_OPT_DECODE_SPLIT_KEYS] // 32) * 32
        assert info["decode_split_keys"] == split
        for it in items:
            if it["kind"] == 1:
                assert it["kv_end"] - it["kv_begin"] <= split


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name + f"_w{w.window}_g{w.num_q_heads // w.num_kv_heads}")
def test_all_decode_path_chunks_every_sequence(w):
    """Path 3: every token in decode items of at most 16 rows (the bf16
    table), long sequences in consecutive chunks; with G above that no decode
    item fits and the prefill kernel keeps the sequences."""
    cu, kv, info, items = plan_for(w, [(RPA_OPT_PATH, 3)])
    check_plan(w, cu, kv, info, items)
    g_ratio = w.num_q_heads // w.num_kv_heads
    limit = 16
    if g_ratio <= limit:
        assert info["num_prefill_items"] == 0
        per = limit // g_ratio
        for it in items:
            if it["split_index"] == 0:
                s = it["seq"]
                # chunks start at multiples of limit / G tokens of their sequence
                assert (it["q_start"] - cu[s]) % per == 0
                assert it["q_count"] == min(per, cu[s + 1] - it["q_start"])
    else:
        assert info["num_decode_items"] == 0


def prefill_keys(items):
    return [it["kv_end"] - it["kv_begin"] for it in items if it["kind"] == 0]


def test_long_prefill_items_are_split_when_they_would_dominate():
    """Mixed step, full causal: the last query tiles of the 4096-token chunk see
    about twice the average key count of a compute unit, so they are cut along
    their key range; the sliding-window and single-chunk workloads keep whole
    items."""
    w = wl.mixed(window=0)
    cu, kv, info, items = plan_for(w)
    check_plan(w, cu, kv, info, items)
    piece = info["prefill_split_keys"]
    assert piece > 0 and piece % 256 == 0
    assert max(prefill_keys(items)) <= 1.5 * piece + 64
    assert any(it["split_group"] >= 0 and it["kind"] == 0 for it in items)
    unsplit = plan_for(w, [(RPA_OPT_PREFILL_SPLIT_KEYS, -1)])
    assert unsplit[2]["prefill_split_keys"] == 0
    assert max(prefill_keys(unsplit[3])) > 1.5 * piece
    for w in [wl.mixed(window=1024), wl.swa_prefill(), wl.global_prefill()]:
        info, items = plan_for(w)[2:]
        assert info["prefill_split_keys"] == 0
        assert all(it["split_group"] == -1 for it in items if it["kind"] == 0)


def test_few_row_prefill_items_split_finer():
    """Single tokens of 32 grouped heads (too many rows for a decode item of
    the bf16 table) go to the prefill kernel with a quarter of its tile's
    rows.  Their key ranges are cut into pieces of the average per
    workgroup slot (two d = 128 prefill workgroups per compute unit), rounded
    up to 128 keys, at least 128; items with full tiles keep the 512-key floor
    (the mixed step above).  With decode items of up to 32 rows the same
    step runs two-block decode items."""
    rng = np.random.default_rng(7)
    w = wl.custom([(1, int(k)) for k in rng.integers(64, 2049, 128)], 32, 1, 128, 128, 0, seed=312)
    cu, kv, info, items = plan_for(w, [(RPA_OPT_DECODE_MAX_ROWS, 32)])
    check_plan(w, cu, kv, info, items)
    assert info["num_prefill_items"] == 0 and all(it["kind"] == 2 for it in items)
    cu, kv, info, items = plan_for(w)
    check_plan(w, cu, kv, info, items)
    assert info["num_decode_items"] == 0
    piece = info["prefill_split_keys"]
    per_slot = sum(k for _, k in w.seqs) / (256 * 2)
    assert piece % 128 == 0 and 128 <= piece < 512
    assert per_slot <= piece < per_slot + 128
    assert max(prefill_keys(items)) <= 1.5 * piece + 64


@pytest.mark.parametrize("piece", [512, 700, 2000])
def test_fixed_prefill_split_keeps_coverage(piece):
    w = wl.custom([(1000, 3000), (3, 40), (700, 700), (1, 900)], 8, 2, 128, 16, 0, 5)
    cu, kv, info, items = plan_for(w, [(RPA_OPT_PREFILL_SPLIT_KEYS, piece)])
    check_plan(w, cu, kv, info, items)
    rounded = -(-max(piece, 512) // 256) * 256
    longest = max(prefill_keys(plan_for(w, [(RPA_OPT_PREFILL_SPLIT_KEYS, -1)])[3]))
    assert info["prefill_split_keys"] == (rounded if longest > 1.5 * rounded else 0)
    assert max(prefill_keys(items)) <= max(1.5 * rounded + 64, longest if longest <= 1.5 * rounded else 0)


def test_decode_selection_rule():
    # bf16 table: q_len * G <= 16 -> decode kernel, more -> prefill
    w = wl.custom([(1, 50), (2, 50), (3, 50), (4, 50), (5, 50)], 8, 1, 256, 128, 0, 9)
    cu, kv, info, items = plan_for(w)
    kinds = {it["seq"]: it["kind"] for it in items}
    assert kinds == {0: 1, 1: 1, 2: 0, 3: 0, 4: 0}
    # the option raises the rows of a decode item: 17..32 -> two-block decode kernel
    kinds = {it["seq"]: it["kind"] for it in plan_for(w, [(RPA_OPT_DECODE_MAX_ROWS, 32)])[3]}
    assert kinds == {0: 1, 1: 1, 2: 2, 3: 2, 4: 0}
    # head size 512 has no two-block decode kernel
    w = wl.custom([(1, 50), (2, 50), (3, 50)], 8, 1, 512, 128, 0, 9)
    kinds = {it["seq"]: it["kind"] for it in plan_for(w, [(RPA_OPT_DECODE_MAX_ROWS, 32)])[3]}
    assert kinds == {0: 1, 1: 1, 2: 0}
    # and a lower cap keeps more sequences on the prefill kernel
    w = wl.custom([(1, 50), (2, 50), (3, 50)], 8, 1, 256, 128, 0, 9)
    kinds = {it["seq"]: it["kind"] for it in plan_for(w, [(RPA_OPT_DECODE_MAX_ROWS, 8)])[3]}
    assert kinds == {0: 1, 1: 0, 2: 0}


# The (head size, group, regime) table the planner follows for a bf16
# cache: for each head size d and group G, a sequence of q_len tokens has
# q_len * G rows; up to 16 rows run the decode kernel (kind 1), more rows the
# prefill kernel (kind 0) with its tile of prefill_rows rows.  (An fp8 cache
# sends 17..32 rows to the two-block decode kernel at d <= 256; the GPU tests
# check that half of the table, whose plans rpa_plan does not expose.)
TABLE_ROWS = {64: 256, 128: 128, 256: 256, 512: 128}


def table_kind(d, rows, fp8=False):
    if rows <= 16:
        return 1
    if fp8 and rows <= 32 and d <= 256:
        return 2
    return 0


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32])
def test_tuning_table(d, g):
    """Every (head size, group) pair in each regime: single-token decode,
    few-token steps (2 and 4 tokens), a short chunk and a long prefill."""
    q_lens = [1, 2, 4, 9, 300]
    w = wl.custom([(q, q + 200) for q in q_lens], g, 1, d, 64, 0, 11)
    cu, kv, info, items = plan_for(w)
    check_plan(w, cu, kv, info, items)
    assert info["prefill_rows"] == TABLE_ROWS[d]
    for s, q in enumerate(q_lens):
        kinds = {it["kind"] for it in items if it["seq"] == s}
        assert kinds == {table_kind(d, q * g)}, (d, g, q, kinds)


def test_prefill_tile_rows_and_longest_first():
    w = wl.swa_prefill(tokens=2000)
    cu, kv, info, items = plan_for(w, [(RPA_OPT_XCD_GROUPS, 0)])
    g_ratio = w.num_q_heads // w.num_kv_heads
    assert all(it["q_count"] * g_ratio <= info["prefill_rows"] for it in items)
    cost = [(it["kv_end"] - it["kv_begin"]) * it["q_count"] for it in items]
    assert cost == sorted(cost, reverse=True)


@pytest.mark.parametrize("w", [wl.swa_prefill(), wl.global_prefill(tokens=3000), wl.mixed(window=0)],
                         ids=["swa", "global3000", "mixed"])
@pytest.mark.parametrize("groups", [8, 3])
def test_chiplet_order_deals_short_runs(w, groups):
    """Launch position b runs on chiplet b mod X.  Each round of 256 positions
    (one workgroup per compute unit) holds the same items as that round of the
    longest-first list; every chiplet takes them in list order, in runs of 4
    consecutive items dealt to the chiplets 0..X-1, then X-1..0, and so on
    (exactly so when a round splits evenly), which keeps the chiplets' work
    within a few percent of each other."""
    key = lambda it: (it["seq"], it["kv_head"], it["q_start"], it["split_index"])
    plain = [key(it) for it in plan_for(w, [(RPA_OPT_XCD_GROUPS, 0)])[3] if it["kind"] == 0]
    cu, kv, info, items = plan_for(w, [(RPA_OPT_XCD_GROUPS, groups)])
    check_plan(w, cu, kv, info, items)
    pre = [it for it in items if it["kind"] == 0]
    got = [key(it) for it in pre]
    rank = {k: i for i, k in enumerate(plain)}
    assert len(got) == len(plain) and len(rank) == len(plain)
    rnd, run = 256, 4
    for r0 in range(0, len(plain), rnd):
        m = min(rnd, len(plain) - r0)
        assert sorted(got[r0:r0 + m]) == sorted(plain[r0:r0 + m])
        for x in range(groups):
            ranks = [rank[got[r0 + pos]] for pos in range(x, m, groups)]
            assert ranks == sorted(ranks)
            if m % (2 * groups * run) == 0:
                runs = [c for c in range(m // run) if (c % groups if (c // groups) % 2 == 0
                                                       else groups - 1 - c % groups) == x]
                assert ranks == [r0 + run * c + i for c in runs for i in range(run)]
    if len(plain) > groups:
        assert got != plain
    if len(plain) >= rnd and groups == 8:
        cost = [0] * groups
        for b, it in enumerate(pre):
            cost[b % groups] += (it["kv_end"] - it["kv_begin"]) * it["q_count"]
        assert max(cost) <= 1.03 * min(cost)


def test_chiplet_order_is_the_default():
    w = wl.swa_prefill()
    default = plan_for(w)[3]
    assert default == plan_for(w, [(RPA_OPT_XCD_GROUPS, 8)])[3]
    assert default != plan_for(w, [(RPA_OPT_XCD_GROUPS, 0)])[3]


def test_auto_split_fills_the_chip():
    w = wl.decode()
    cu, kv, info, items = plan_for(w)
    assert info["num_decode_items"] >= 256       # more workgroups than compute units
    assert info["decode_split_keys"] % 128 == 0
    assert info["num_partials"] == sum(it["split_group"] >= 0 for it in items)


def test_plan_is_deterministic():
    w = wl.mixed(window=1024)
    a = plan_for(w)
    b = plan_for(w)
    assert a[2] == b[2] and a[3] == b[3]


def test_fp8_staging_list_covers_every_page_prefill_items_read(tmp_path):
    """The planner's fp8 staging list (internal, not exposed through the C
    ABI) checked by a small C++ program on random ragged batches, built here
    with g++ against the planner source (address and UB sanitizers on)."""
    import os
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "ragged_paged_attention_forward_amd", "csrc")
    exe = str(tmp_path / "plan_stage_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-fsanitize=address,undefined", "-I", os.path.join(root, "include"),
                    "-I", csrc, os.path.join(root, "tests", "plan_stage_check.cpp"),
                    os.path.join(csrc, "rpa_plan.cpp"), "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
