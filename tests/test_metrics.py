"""Pins of the throughput accounting (CPU only): brute force over the oracle's
visibility rule, and the figures the pages print (tests/golden/page_figures.json)."""
import json
import math
import os

import numpy as np
import pytest

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from ragged_paged_attention_forward_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _cases():
    rng = np.random.default_rng(0)
    out = []
    for window in (0, 1, 3, 17, 64, 1000):
        seqs = []
        for _ in range(6):
            kv = int(rng.integers(0, 200))
            q = int(rng.integers(0, kv + 1))
            seqs.append((q, kv))
        out.append((seqs, window))
    return out


@pytest.mark.parametrize("seqs,window", _cases())
def test_pairs_and_unique_keys_match_brute_force(seqs, window):
    pairs = 0
    keys = 0
    for q, kv in seqs:
        m = ora.visible(q, kv, window)
        pairs += int(m.sum())
        keys += int(m.any(axis=0).sum()) if q else 0
    assert metrics.visible_pairs(seqs, window) == pairs
    assert metrics.unique_keys(seqs, window) == keys


def test_named_workload_pair_counts():
    # brute force the visibility rule for the fixed-shape workloads
    for w in (wl.tiny(), wl.swa_prefill(tokens=3000), wl.global_prefill(tokens=2000)):
        brute = sum(int(ora.visible(q, kv, w.window).sum()) for q, kv in w.seqs)
        assert metrics.visible_pairs(w.seqs, w.window) == brute
    # long shapes: closed forms of a full causal triangle and a clipped band
    assert metrics.visible_pairs([(8192, 8192)], 0) == 8192 * 8193 // 2
    assert metrics.visible_pairs([(8192, 8192)], 1024) == 1024 * 1025 // 2 + (8192 - 1024) * 1024


def test_flops_count_matches_training_table():
    fig = json.load(open(GOLDEN))["training_flops_dot_product_attention"]
    d, hq = 256, 8
    per_pair_per_head = metrics.flops([(1, 1)], 0, hq, d) / hq
    assert per_pair_per_head == fig["coefficient"] * d / fig["training_multiplier"]


def test_kv_fetches_per_key_page_figure():
    fig = json.load(open(GOLDEN))["kv_fetches_per_key"]
    f = metrics.kv_fetches_per_key(fig["window"], fig["query_block"])
    assert fig["at_least"] <= f < fig["less_than"]


@pytest.mark.parametrize("window,block", [(1024, 32), (1024, 512), (100, 7), (64, 64)])
def test_kv_fetches_per_key_brute_force(window, block):
    """Average, over keys far from both ends, of the query blocks that want the key."""
    n = 8 * window + 5 * block
    counts = []
    for key in range(2 * window, n - 2 * window):
        first_q, last_q = key, key + window - 1   # queries that see this key
        counts.append(last_q // block - first_q // block + 1)
    assert math.isclose(np.mean(counts), metrics.kv_fetches_per_key(window, block), rel_tol=2e-2)


def test_decode_intensity_page_figure():
    fig = json.load(open(GOLDEN))["decode_intensity_flop_per_byte"]
    hq, hkv, d = fig["num_q_heads"], fig["num_kv_heads"], fig["head_dim"]
    for kv in (64, 140, 640, 4096):
        seqs = [(1, kv)] * 32
        kv_only = metrics.flops(seqs, 0, hq, d) / metrics.kv_bytes(seqs, 0, hkv, d)
        assert kv_only == pytest.approx(fig["approx"])
        with_qo = metrics.flops(seqs, 0, hq, d) / (metrics.kv_bytes(seqs, 0, hkv, d) +
                                                  metrics.qo_bytes(seqs, hq, d))
        assert 0.85 * fig["approx"] < with_qo <= fig["approx"]


def test_attention_intensity_formula_for_decode():
    fig = json.load(open(GOLDEN))["attention_intensity_formula"]
    for t, s, g in fig["cases"]:
        if t != 1:
            continue   # causal masking breaks the all-pairs formula for T > 1
        hq, hkv, d = g, 1, 128
        seqs = [(1, s)]
        ai = metrics.flops(seqs, 0, hq, d) / (metrics.kv_bytes(seqs, 0, hkv, d) +
                                              metrics.qo_bytes(seqs, hq, d))
        assert ai == pytest.approx(t * s * g / (t * g + s))
