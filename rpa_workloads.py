"""Seeded synthetic inputs for ragged paged attention.

This module only *builds inputs*: token counts, page tables and bf16 tensors
drawn from N(0, 1).  It holds none of the attention arithmetic, so both the
CPU oracle (``oracle/``) and the GPU path (``ragged_paged_attention_forward_amd``)
can be fed from it without sharing any of the method's code.

Workloads follow the shapes the pages describe:

* decode with Gemma-2B-like multi-query heads (8 query heads sharing one KV
  head of width 256, 128-token pages) -- "Pallas Kernel: vLLM on TPU ...",
  section S3 (batch scaling) and S7 (block-size tuning);
* an 8192-token prefill through a sliding-window (1024) layer and through a
  global layer -- "Chasing speed of light on TPU v6e", section Attention;
* a chunked-prefill step with an 8192-token budget mixing prefill chunks with
  single-token decodes -- "Pallas Kernel: vLLM on TPU ...", environment
  section (chunked prefill, prefix cache), and "TPU Deep Dive" chapter 8
  (flattened token batch plus per-sequence metadata).

Layouts (all row-major):
  q          [T, Hq, D]        bf16, T = cu_q_lens[-1]
  k_pages    [P, B, Hkv, D]    bf16, P = pages in the pool (incl. one trap page)
  v_pages    [P, B, Hkv, D]    bf16
  page_table [S, max_pages]    int32, unused entries hold the trap page id
  cu_q_lens  [S + 1]           int32, cu_q_lens[0] = 0, non-decreasing
  kv_lens    [S]               int32, kv_lens[s] >= q_len(s)

Draw order from ``np.random.default_rng(seed)``: random kv lengths, page
permutation, Q, K pool, V pool.  Values are float32 normals rounded to bf16
with round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch


@dataclass
class Workload:
    """Shape of one attention call: per-sequence (q_len, kv_len) plus heads."""

    name: str
    seqs: List[Tuple[int, int]]          # (q_len, kv_len) per sequence
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window: int = 0                      # 0: full causal
    seed: int = 0
    extra_pages_per_seq: int = 0         # page-table slack beyond what is needed
    description: str = ""
    length_draw: Tuple[int, ...] = ()    # (low, high_exclusive, count) drawn first, if any

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def num_seqs(self) -> int:
        return len(self.seqs)

    @property
    def total_q(self) -> int:
        return int(sum(q for q, _ in self.seqs))

    def pages_needed(self) -> List[int]:
        b = self.page_size
        return [(kv + b - 1) // b for _, kv in self.seqs]

    @property
    def max_pages_per_seq(self) -> int:
        need = self.pages_needed()
        return (max(need) if need else 0) + self.extra_pages_per_seq or 1


# ---------------------------------------------------------------------------
# The five named workloads.  Random kv lengths are drawn first from the seed.
# ---------------------------------------------------------------------------

SEEDS = {"tiny": 101, "decode": 102, "swa_prefill": 103, "global_prefill": 104,
         "mixed": 105, "mixed_swa": 105}


def tiny(seed: int = SEEDS["tiny"]) -> Workload:
    """2 sequences, q_len = kv_len = 37 and 100; 4 q heads on 1 KV head, d 64, B 16."""
    return Workload("tiny", [(37, 37), (100, 100)], 4, 1, 64, 16, 0, seed,
                    description="tiny prefill: q=kv in {37,100}, Hq4/Hkv1, d64, B16, causal")


def decode(seed: int = SEEDS["decode"], num_seqs: int = 128) -> Workload:
    """128 single-token decodes, kv_len ~ U[64, 640]; 8 q heads on 1 KV head, d 256, B 128."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 641, num_seqs)
    return Workload("decode", [(1, int(k)) for k in kv], 8, 1, 256, 128, 0, seed,
                    description=f"decode batch: {num_seqs} x (q 1, kv U[64,640]), "
                                "Hq8/Hkv1, d256, B128",
                    length_draw=(64, 641, num_seqs))


def swa_prefill(seed: int = SEEDS["swa_prefill"], tokens: int = 8192,
                num_q_heads: int = 16, num_kv_heads: int = 8) -> Workload:
    """One 8192-token causal prefill through a window of 1024; 16 q / 8 KV heads, d 256."""
    return Workload("swa_prefill", [(tokens, tokens)], num_q_heads, num_kv_heads, 256, 128,
                    1024, seed,
                    description=f"sliding-window prefill: 1 x {tokens}, W1024, "
                                f"Hq{num_q_heads}/Hkv{num_kv_heads}, d256, B128")


def global_prefill(seed: int = SEEDS["global_prefill"], tokens: int = 8192,
                   num_q_heads: int = 16, num_kv_heads: int = 2) -> Workload:
    """One 8192-token full-causal prefill; 16 q / 2 KV heads, d 512."""
    return Workload("global_prefill", [(tokens, tokens)], num_q_heads, num_kv_heads, 512, 128,
                    0, seed,
                    description=f"global prefill: 1 x {tokens}, causal, "
                                f"Hq{num_q_heads}/Hkv{num_kv_heads}, d512, B128")


def mixed(seed: int = SEEDS["mixed"], window: int = 0, num_decodes: int = 512) -> Workload:
    """Chunked-prefill step: 4 chunks (q, prior) = (4096,0) (2048,1024) (1024,3072)
    (512,512) followed by 512 decodes with kv_len ~ U[64, 1024]; 8 q / 1 KV, d 256."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1025, num_decodes)
    chunks = [(4096, 4096), (2048, 3072), (1024, 4096), (512, 1024)]
    seqs = chunks + [(1, int(k)) for k in kv]
    name = "mixed" if window == 0 else "mixed_swa"
    return Workload(name, seqs, 8, 1, 256, 128, window, seed,
                    description=f"mixed step: 4 prefill chunks + {num_decodes} decodes, "
                                f"Hq8/Hkv1, d256, B128, W{window}",
                    length_draw=(64, 1025, num_decodes))


def swa_prefill_share8(seed: int = SEEDS["swa_prefill"]) -> Workload:
    """One GPU's share of swa_prefill split by KV head over 8 GPUs: 2 q / 1 KV head."""
    w = swa_prefill(seed, num_q_heads=2, num_kv_heads=1)
    w.name = "swa_prefill_share8"
    w.description += " (one GPU's share of 8)"
    return w


def global_prefill_share2(seed: int = SEEDS["global_prefill"]) -> Workload:
    """One GPU's share of global_prefill split by KV head over 2 GPUs: 8 q / 1 KV head."""
    w = global_prefill(seed, num_q_heads=8, num_kv_heads=1)
    w.name = "global_prefill_share2"
    w.description += " (one GPU's share of 2)"
    return w


def by_name(name: str) -> Workload:
    table = {"tiny": tiny, "decode": decode, "swa_prefill": swa_prefill,
             "global_prefill": global_prefill, "mixed": lambda: mixed(window=0),
             "mixed_swa": lambda: mixed(window=1024), "swa_prefill_share8": swa_prefill_share8,
             "global_prefill_share2": global_prefill_share2}
    return table[name]()


# ---------------------------------------------------------------------------
# Tensor construction
# ---------------------------------------------------------------------------

@dataclass
class Inputs:
    """Host (CPU) tensors of one call.  ``trap_page`` is the pool's extra page."""

    workload: Workload
    q: torch.Tensor            # [T, Hq, D] bf16
    k_pages: torch.Tensor      # [P, B, Hkv, D] bf16
    v_pages: torch.Tensor      # [P, B, Hkv, D] bf16
    page_table: torch.Tensor   # [S, max_pages] int32
    cu_q_lens: torch.Tensor    # [S + 1] int32
    kv_lens: torch.Tensor      # [S] int32
    trap_page: int
    window: int
    scale: float
    poisoned: bool = False

    def to(self, device) -> "Inputs":
        return Inputs(self.workload, self.q.to(device), self.k_pages.to(device),
                      self.v_pages.to(device), self.page_table.to(device),
                      self.cu_q_lens, self.kv_lens, self.trap_page, self.window,
                      self.scale, self.poisoned)


def _bf16_normal(rng: np.random.Generator, shape) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def make_inputs(w: Workload, seed: Optional[int] = None, poison: bool = False,
                shuffle: bool = True) -> Inputs:
    """Draw the tensors of workload ``w``.

    ``poison`` fills every page slot past a sequence's kv_len and the whole trap
    page with NaN, so a kernel that reads them shows it in its output.
    ``shuffle`` False gives the identity page assignment (sequence-major).
    """
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    # Random kv lengths were already drawn into the workload from the same seed;
    # draw them again so the stream position matches the documented draw order
    # before the page permutation.
    if w.length_draw:
        rng.integers(*w.length_draw)
    need = w.pages_needed()
    n_pages = int(sum(need))
    perm = rng.permutation(n_pages) if shuffle else np.arange(n_pages)
    trap = n_pages
    s_count = w.num_seqs
    max_pages = w.max_pages_per_seq
    pt = np.full((s_count, max_pages), trap, dtype=np.int32)
    cursor = 0
    for s, n in enumerate(need):
        pt[s, :n] = perm[cursor:cursor + n]
        cursor += n
    t_q = w.total_q
    q = _bf16_normal(rng, (t_q, w.num_q_heads, w.head_dim))
    pool_shape = (n_pages + 1, w.page_size, w.num_kv_heads, w.head_dim)
    k_pages = _bf16_normal(rng, pool_shape)
    v_pages = _bf16_normal(rng, pool_shape)
    cu = np.zeros(s_count + 1, dtype=np.int32)
    cu[1:] = np.cumsum([ql for ql, _ in w.seqs])
    kv = np.array([kl for _, kl in w.seqs], dtype=np.int32)
    if poison:
        nan = float("nan")
        k_pages[trap] = nan
        v_pages[trap] = nan
        for s, (_, kl) in enumerate(w.seqs):
            n = need[s]
            if n == 0:
                continue
            tail = kl - (n - 1) * w.page_size     # slots used in the last page
            last = int(pt[s, n - 1])
            k_pages[last, tail:] = nan
            v_pages[last, tail:] = nan
    return Inputs(w, q, k_pages, v_pages, torch.from_numpy(pt), torch.from_numpy(cu),
                  torch.from_numpy(kv), trap, w.window, w.scale, poison)


@dataclass
class Fp8Inputs:
    """An fp8 KV cache drawn from a bf16 call's tensors: the pools hold OCP FP8
    E4M3 bytes [P, B, Hkv, D] (uint8) and each KV head has one float32 scale
    for K and one for V.  ``base`` keeps the bf16 tensors (q, page table,
    lengths) the call shares."""

    base: Inputs
    k_pages: torch.Tensor   # [P, B, Hkv, D] uint8
    v_pages: torch.Tensor   # [P, B, Hkv, D] uint8
    k_scales: torch.Tensor  # [Hkv] float32
    v_scales: torch.Tensor  # [Hkv] float32

    def to(self, device) -> "Fp8Inputs":
        return Fp8Inputs(self.base.to(device), self.k_pages.to(device), self.v_pages.to(device),
                         self.k_scales.to(device), self.v_scales.to(device))


NAN_E4M3 = 0x7F   # the E4M3 NaN byte


def _to_e4m3(pool: torch.Tensor, rng: np.random.Generator) -> Tuple[torch.Tensor, torch.Tensor]:
    """Bytes and per-KV-head scales of a [P, B, Hkv, D] pool: head g gets the
    scale max|x_g| / 448 times a factor drawn from [1, 4) (so heads differ and
    no value saturates); bytes are torch's round-to-nearest E4M3 of x / scale."""
    x = pool.to(torch.float32)
    amax = x.abs().amax(dim=(0, 1, 3)).clamp_min(1e-3)
    factor = torch.from_numpy(rng.uniform(1.0, 4.0, size=x.shape[2]).astype(np.float32))
    scales = (amax / 448.0 * factor).to(torch.float32)
    codes = (x / scales.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scales


def make_fp8_inputs(w: Workload, seed: Optional[int] = None, poison: bool = False,
                    shuffle: bool = True) -> Fp8Inputs:
    """The tensors of ``make_inputs`` with the K and V pools held in fp8.

    ``poison`` fills every page slot past a sequence's kv_len and the whole trap
    page with the E4M3 NaN byte."""
    base = make_inputs(w, seed, poison=False, shuffle=shuffle)
    rng = np.random.default_rng((w.seed if seed is None else seed) + 104729)
    k8, ks = _to_e4m3(base.k_pages, rng)
    v8, vs = _to_e4m3(base.v_pages, rng)
    if poison:
        k8[base.trap_page] = NAN_E4M3
        v8[base.trap_page] = NAN_E4M3
        need = w.pages_needed()
        for s, (_, kl) in enumerate(w.seqs):
            n = need[s]
            if n == 0:
                continue
            tail = kl - (n - 1) * w.page_size
            last = int(base.page_table[s, n - 1])
            k8[last, tail:] = NAN_E4M3
            v8[last, tail:] = NAN_E4M3
        base.poisoned = True
    return Fp8Inputs(base, k8, v8, ks, vs)


def custom(seqs: Sequence[Tuple[int, int]], num_q_heads: int, num_kv_heads: int,
           head_dim: int, page_size: int, window: int = 0, seed: int = 0,
           extra_pages_per_seq: int = 0, name: str = "custom") -> Workload:
    """A free-form workload for tests (no random lengths drawn)."""
    return Workload(name, [(int(a), int(b)) for a, b in seqs], num_q_heads, num_kv_heads,
                    head_dim, page_size, window, seed, extra_pages_per_seq)


def sample_rows(t_q: int, count: int, seed: int, must: Sequence[int] = ()) -> np.ndarray:
    """Seeded sample of output token rows (always including ``must``)."""
    rng = np.random.default_rng(seed + 7919)
    pick = set(int(x) for x in must if 0 <= x < t_q)
    if t_q > 0:
        pick.update(int(x) for x in rng.choice(t_q, size=min(count, t_q), replace=False))
    return np.array(sorted(pick), dtype=np.int64)
