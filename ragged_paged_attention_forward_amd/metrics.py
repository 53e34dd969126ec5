"""Algorithmic work of one ragged paged attention call (for throughput reporting).

Counting follows the pages' roofline accounting ("Chasing speed of light on TPU
v6e", footnote 5 of section Attention): every visible (query, key) pair costs
two d-length dot products per query head -- q.k and p.v -- i.e. 4*d FLOPs; an
ideal kernel moves Q, K, V and O through HBM exactly once.  "TPU Deep Dive",
chapter 4 gives the same per-head count (dot-product attention is 4x of the
forward-pass share of 12*B*T*S*N*H training FLOPs) and the intensity
AI = T*S*G / (T*G + S), about G for decode.

Bytes are *unique* bytes: Q and O once, and every key/value row that at least
one query of its sequence can see, once (re-reads and page tails excluded).
"""
from __future__ import annotations

from typing import Iterable, Tuple

BF16 = 2


def _rows(q_len: int, kv_len: int):
    first = kv_len - q_len
    return range(first, kv_len)


def visible_keys(pos: int, window: int) -> int:
    """Keys visible from position ``pos``: 0..pos, clipped to the last ``window``."""
    return min(pos + 1, window) if window > 0 else pos + 1


def visible_pairs(seqs: Iterable[Tuple[int, int]], window: int) -> int:
    """Visible (query, key) pairs per query head, summed over sequences (closed form)."""
    total = 0
    for q_len, kv_len in seqs:
        if q_len == 0:
            continue
        first = kv_len - q_len
        if window <= 0:
            # sum_{p=first}^{kv_len-1} (p + 1)
            total += (kv_len * (kv_len + 1) - first * (first + 1)) // 2
        else:
            # positions p < window see p+1 keys, the rest see `window`
            lo_end = min(kv_len, window)       # positions [first, lo_end) are unclipped
            if first < lo_end:
                total += (lo_end * (lo_end + 1) - first * (first + 1)) // 2
                total += (kv_len - lo_end) * window
            else:
                total += q_len * window
    return total


def unique_keys(seqs: Iterable[Tuple[int, int]], window: int) -> int:
    """Key rows of all sequences seen by at least one query of their sequence."""
    total = 0
    for q_len, kv_len in seqs:
        if q_len == 0:
            continue
        first = kv_len - q_len
        lo = max(0, first - window + 1) if window > 0 else 0
        total += kv_len - lo
    return total


def flops(seqs, window: int, num_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * num_q_heads * visible_pairs(seqs, window)


def kv_bytes(seqs, window: int, num_kv_heads: int, head_dim: int) -> int:
    """Unique K plus V bytes read (bf16)."""
    return 2 * BF16 * head_dim * num_kv_heads * unique_keys(seqs, window)


def qo_bytes(seqs, num_q_heads: int, head_dim: int) -> int:
    t = sum(q for q, _ in seqs)
    return 2 * BF16 * t * num_q_heads * head_dim


def total_bytes(seqs, window: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                page_size: int = 0) -> int:
    """Q + O + unique K/V + metadata (page-table entries and the two length arrays)."""
    meta = 0
    for q_len, kv_len in seqs:
        meta += 4 * 2
        if page_size:
            meta += 4 * ((kv_len + page_size - 1) // page_size)
    return qo_bytes(seqs, num_q_heads, head_dim) + kv_bytes(seqs, window, num_kv_heads, head_dim) + meta


def kv_fetches_per_key(window: int, query_block: int) -> float:
    """How many query blocks want a given key in a long sliding-window prefill.

    A key is wanted by the ``window`` queries following it (itself included);
    they straddle ceil(window / block) blocks when the key sits at a block
    boundary and one more otherwise: on average (window - 1) / block + 1.
    """
    return (window - 1) / query_block + 1


def decode_intensity(kv_len: int, group: int) -> float:
    """FLOP per K/V byte of a one-token decode: 4*d*G*kv / (2*2*d*kv) = G."""
    d = 1
    return (4 * d * group * kv_len) / (2 * BF16 * d * kv_len)
