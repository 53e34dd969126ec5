"""Plain fp64 CPU oracle for ragged paged attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it, and it
shares no code with the GPU library: it is the plain definition written out,
slow on purpose, so that a reader can check it against the pages by eye.

What it computes (the pages' method, read plainly):

* The step's query tokens of all sequences sit in one flattened array; each
  sequence's slice is given by cumulative query lengths, and its true KV length
  by per-sequence metadata ("TPU Deep Dive", chapter 8, "Continuous batching
  with static shapes": flattened token batch + per-sequence metadata; true
  lengths handled inside the kernel).
* A sequence's keys and values live in fixed-size pages found through its page
  table ("Pallas Kernel: vLLM on TPU ...", environment section and S3: KV held
  in 128-token blocks).  Un-paging is a pure gather: key t of sequence s is slot
  t mod B of page ``page_table[s][t div B]``.
* Query tokens are the *last* q_len positions of the sequence: row r sits at
  absolute position p = kv_len - q_len + r (chunked prefill on top of earlier
  context, same page, environment section).
* Several query heads share one KV head ("TPU Deep Dive", chapter 4, "Shape
  on TPU": KV heads; "Pallas Kernel ...", S3: 8 query heads share 1 KV head).
  Reading: contiguous groups, query head h uses KV head h // G, G = Hq / Hkv.
* Causal attention, optionally through a sliding window: in a sliding-window
  layer a key is wanted by the W queries that follow it ("Chasing speed of
  light on TPU v6e", section Attention).  Reading: with W > 0, query position p
  sees keys j with p - W + 1 <= j <= p (W keys counting itself); W = 0 means
  full causal, j <= p.
* Each (query, key) pair costs a q.k dot product and a p.v product per query
  head -- two matmuls per head -- and the normalised scores never leave the
  chip ("Chasing speed of light on TPU v6e", footnote 5 of section Attention).
  Written out: out = softmax(scale * Q K^T + mask) V per sequence and head, with
  mask = 0 on visible pairs and -inf elsewhere.

Everything is done in float64 on values converted exactly from the bf16 inputs.
Nothing here is blocked, fused or reordered: rows are processed in groups of at
most ``ROW_BLOCK`` only to bound memory, which is exact because rows of a
softmax are independent.

An fp8 KV cache ("TPU Deep Dive", chapter 7, quantization levers: KV held in
fp8 halves the dominant long-context read; "Pallas Kernel: vLLM on TPU ...",
S5: a working cache quantization doubles the cache's token capacity) is read
here as the pages leave it open: every stored K or V element is one byte in
the OCP FP8 E4M3 format, and each KV head has one float32 scale for K and one
for V; the value an element stands for is its E4M3 value times its head's
scale.  ``forward_fp8_rows`` dequantizes exactly that way and then computes
the same attention as ``forward_rows``.  New tokens enter such a cache as
``quantize_e4m3`` of their value divided by the head's scale in float32 (the
nearest code, ties to even, saturating at 448): ``append_kv_fp8``.

Every function below is pinned by ``tests/test_oracle.py`` (brute force, a
library routine, closed forms, invariants, and for ``append_kv`` a hand-worked
case and a round trip through generated pages); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

ROW_BLOCK = 1024


def as_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (any float dtype incl. bf16) or array to float64."""
    if hasattr(x, "detach"):
        import torch  # CPU only; plain dtype conversion
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def as_i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def unpage(pages: np.ndarray, table_row: np.ndarray, kv_len: int, page_size: int) -> np.ndarray:
    """Gather the first ``kv_len`` token rows of one sequence from the page pool.

    pages: [P, B, Hkv, D]; table_row: the sequence's page-table row.
    Returns [kv_len, Hkv, D]: row t = pages[table_row[t // B], t % B].
    """
    out = np.empty((kv_len,) + pages.shape[2:], dtype=np.float64)
    for t in range(kv_len):
        out[t] = pages[int(table_row[t // page_size]), t % page_size]
    return out


def visible(q_len: int, kv_len: int, window: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(rows), kv_len]: True where query row r may attend to key j.

    Row r is at position p = kv_len - q_len + r; key j is visible iff j <= p and,
    for a window W > 0, j >= p - W + 1.
    """
    if rows is None:
        rows = np.arange(q_len)
    p = (kv_len - q_len + np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    ok = j <= p
    if window > 0:
        ok &= j >= p - window + 1
    return ok


def softmax_rows(scores: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax of ``scores`` where masked entries count as -inf."""
    s = np.where(mask, scores, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def _check_metadata(cu: np.ndarray, kv: np.ndarray, num_q_heads: int, num_kv_heads: int,
                    window: int) -> None:
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    if window < 0:
        raise ValueError("window must be >= 0")
    if cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_q_lens must start at 0 and be non-decreasing")
    if np.any(np.diff(cu) > kv):
        raise ValueError("q_len may not exceed kv_len")


def sequence_probs(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, window: int,
                   scale: float, seq: int, head: int) -> np.ndarray:
    """Debug hook: the [q_len, kv_len] probability matrix P of one sequence and query head."""
    qf, kf = as_f64(q), as_f64(k_pages)
    pt, cu, kv = as_i64(page_table), as_i64(cu_q_lens), as_i64(kv_lens)
    hq, hkv = qf.shape[1], kf.shape[2]
    g = head // (hq // hkv)
    q_len, kv_len = int(cu[seq + 1] - cu[seq]), int(kv[seq])
    k_s = unpage(kf, pt[seq], kv_len, kf.shape[1])
    q_h = qf[cu[seq]:cu[seq + 1], head, :]
    s = scale * (q_h @ k_s[:, g, :].T)
    return softmax_rows(s, visible(q_len, kv_len, window))


def forward_rows(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, window: int,
                 scale: float, token_rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Oracle output for the selected flattened token rows (all of them if None).

    Returns float64 [len(token_rows), Hq, D] in the order of ``token_rows``.
    """
    qf = as_f64(q)
    kf = as_f64(k_pages)
    vf = as_f64(v_pages)
    pt = as_i64(page_table)
    cu = as_i64(cu_q_lens)
    kv = as_i64(kv_lens)
    t_total, hq, d = qf.shape
    hkv, b = kf.shape[2], kf.shape[1]
    _check_metadata(cu, kv, hq, hkv, window)
    group = hq // hkv
    if token_rows is None:
        token_rows = np.arange(t_total)
    token_rows = np.asarray(list(token_rows), dtype=np.int64)
    out = np.full((len(token_rows), hq, d), np.nan, dtype=np.float64)
    # which sequence owns each requested row
    owner = np.searchsorted(cu, token_rows, side="right") - 1
    for s in np.unique(owner):
        s = int(s)
        sel = np.nonzero(owner == s)[0]
        local = token_rows[sel] - cu[s]
        q_len, kv_len = int(cu[s + 1] - cu[s]), int(kv[s])
        k_s = unpage(kf, pt[s], kv_len, b)
        v_s = unpage(vf, pt[s], kv_len, b)
        for lo in range(0, len(sel), ROW_BLOCK):
            blk = slice(lo, lo + ROW_BLOCK)
            rows = local[blk]
            mask = visible(q_len, kv_len, window, rows)
            for h in range(hq):
                g = h // group
                q_h = qf[token_rows[sel[blk]], h, :]
                scores = scale * (q_h @ k_s[:, g, :].T)
                p = softmax_rows(scores, mask)
                out[sel[blk], h, :] = p @ v_s[:, g, :]
    return out


def forward(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, window: int,
            scale: float) -> np.ndarray:
    """Full oracle output, float64 [T, Hq, D]."""
    return forward_rows(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, window, scale)


def append_kv(k_pages, v_pages, page_table, cu_q_lens, kv_lens, k_new, v_new):
    """The step's new keys and values written into their pages, as the pages'
    kernel does within the attention call ("TPU Deep Dive", chapter 8: ragged
    paged attention handles true lengths in the kernel, with a fused KV write).

    Token t of sequence s (cu[s] <= t < cu[s+1]) is at position
    p = kv_len_s - q_len_s + (t - cu[s]) (the step's tokens are the last q_len
    positions); its rows k_new[t], v_new[t] (all KV heads) go to slot p mod B of
    page page_table[s][p div B].  Works on numpy arrays or CPU torch tensors of
    any dtype (bf16 included) and returns new arrays, the inputs untouched:
    a pure copy, so every written value keeps its bits.
    """
    def copy(x):
        return x.clone() if hasattr(x, "clone") else np.array(x, copy=True)

    k_out, v_out = copy(k_pages), copy(v_pages)
    cu, kv, table = as_i64(cu_q_lens), as_i64(kv_lens), as_i64(page_table)
    page_size = k_pages.shape[1]
    for s in range(len(kv)):
        q_len = int(cu[s + 1] - cu[s])
        for r in range(q_len):
            t = int(cu[s]) + r
            p = int(kv[s]) - q_len + r
            page, slot = int(table[s, p // page_size]), p % page_size
            k_out[page, slot] = k_new[t]
            v_out[page, slot] = v_new[t]
    return k_out, v_out


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each OCP FP8 E4M3 byte: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits.  Exponent field e > 0: (1 + m/8) * 2^(e - 7);
    e = 0: subnormal, (m/8) * 2^-6.  The all-ones magnitude 0x7f (either sign)
    is NaN and there is no infinity, so the largest finite value is
    0x7e = 1.75 * 2^8 = 448."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def dequantize_kv(pages, scales) -> np.ndarray:
    """float64 values of an fp8 page pool: ``pages`` holds E4M3 bytes
    [P, B, Hkv, D] (uint8 array or tensor), ``scales`` one float per KV head;
    element (.., g, :) stands for e4m3_value(byte) * scales[g]."""
    codes = pages.detach().cpu().numpy() if hasattr(pages, "detach") else np.asarray(pages)
    sc = as_f64(scales).reshape(1, 1, -1, 1)
    return e4m3_value(codes) * sc


def quantize_e4m3(x) -> np.ndarray:
    """E4M3 byte of each float32 value: the finite code nearest to x, ties to
    the code with an even last mantissa bit; values beyond +-448 take +-448
    (the largest finite code), NaN gives 0x7f; the sign of zero is kept.
    Done by search over the code values, not by bit manipulation."""
    xs = np.asarray(x, dtype=np.float32).astype(np.float64).ravel()
    pos_codes = np.arange(0x7F)                       # 0x00 .. 0x7e: 0 .. 448
    pos_vals = e4m3_value(pos_codes)
    out = np.empty(xs.shape, dtype=np.uint8)
    for i, v in enumerate(xs):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        a = min(abs(v), 448.0)
        d = np.abs(pos_vals - a)
        best = np.nonzero(d == d.min())[0]
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        neg = v < 0 or (v == 0 and np.signbit(v))
        out[i] = c | (0x80 if neg else 0)
    return out.reshape(np.shape(x))


def append_kv_fp8(k_pages, v_pages, k_scales, v_scales, page_table, cu_q_lens, kv_lens, k_new, v_new):
    """The step's new keys and values written into an fp8 cache: each new
    element is divided by its KV head's scale in float32 and stored as
    ``quantize_e4m3`` of that quotient, at the slots ``append_kv`` uses.
    k_pages / v_pages are uint8 arrays or tensors; returns new uint8 arrays."""
    def codes(new, scales):
        x = as_f64(new).astype(np.float32)
        sc = as_f64(scales).astype(np.float32).reshape(1, -1, 1)
        return quantize_e4m3(x / sc)
    kp = k_pages.cpu().numpy() if hasattr(k_pages, "cpu") else np.asarray(k_pages)
    vp = v_pages.cpu().numpy() if hasattr(v_pages, "cpu") else np.asarray(v_pages)
    return append_kv(kp, vp, page_table, cu_q_lens, kv_lens, codes(k_new, k_scales), codes(v_new, v_scales))


def forward_fp8_rows(q, k_pages, v_pages, k_scales, v_scales, page_table, cu_q_lens, kv_lens,
                     window: int, scale: float, token_rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Attention over an fp8 KV cache: the pools are dequantized (``dequantize_kv``)
    and the result is ``forward_rows`` of those values."""
    return forward_rows(q, dequantize_kv(k_pages, k_scales), dequantize_kv(v_pages, v_scales), page_table,
                        cu_q_lens, kv_lens, window, scale, token_rows)


def forward_inputs(inp, token_rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Convenience wrapper over an ``rpa_workloads.Inputs`` bundle."""
    return forward_rows(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                        inp.kv_lens, inp.window, inp.scale, token_rows)
