"""Helpers shared by the GPU tests: run the HIP path, compare with the oracle."""
import numpy as np
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def gpu_available() -> bool:
    return torch.cuda.is_available()


def make_attn(w: wl.Workload, max_num_seqs=None, max_q_tokens=None):
    from ragged_paged_attention_forward_amd import RaggedPagedAttention
    return RaggedPagedAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                max_num_seqs or max(1, w.num_seqs), w.max_pages_per_seq,
                                max_q_tokens or max(1, w.total_q))


def run_gpu(attn, inp: wl.Inputs, window=None, device="cuda") -> torch.Tensor:
    d = inp.to(device)
    out = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, inp.cu_q_lens, inp.kv_lens,
                       inp.window if window is None else window, inp.scale)
    torch.cuda.synchronize()
    return out


def compare(got: torch.Tensor, ref: np.ndarray, rows=None, label=""):
    """Element-wise parity: max-abs <= 2e-2, mean-abs <= 2e-3, no NaN."""
    g = got.detach().to("cpu", torch.float64).numpy()
    if rows is not None:
        g = g[np.asarray(rows)]
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return 0.0, 0.0
    nan = ~np.isfinite(g)
    assert not nan.any(), f"{label}: {int(nan.sum())} non-finite outputs, first at {np.argwhere(nan)[0]}"
    err = np.abs(g - ref)
    mx = float(err.max())
    mean = float(err.mean())
    loc = np.unravel_index(int(err.argmax()), err.shape)
    assert mx <= MAX_ABS, f"{label}: max-abs {mx:.3e} at {loc} (got {g[loc]:.5f} want {ref[loc]:.5f})"
    assert mean <= MEAN_ABS, f"{label}: mean-abs {mean:.3e}"
    return mx, mean


def oracle_rows(inp: wl.Inputs, rows=None) -> np.ndarray:
    return ora.forward_inputs(inp, rows)


def bitwise_mismatch(got: torch.Tensor, want: torch.Tensor, inp: wl.Inputs, label="") -> str:
    """'' when got equals want bit for bit; otherwise a report of the token
    rows that differ (their sequences, how many hold NaN) and of both
    tensors' error against the oracle on a few of them, so that a failure
    names the wrong side."""
    if torch.equal(got, want):
        return ""
    differ = (got.view(torch.int16) != want.view(torch.int16)).flatten(1).any(1).nonzero().flatten().cpu().numpy()
    cu = inp.cu_q_lens.numpy()
    seqs = sorted({int(np.searchsorted(cu, t, side="right") - 1) for t in differ})
    nan_rows = int(torch.isnan(got[torch.from_numpy(differ).to(got.device)]).flatten(1).any(1).sum())
    rows = differ[:: max(1, len(differ) // 6)][:6]
    ref = oracle_rows(inp, rows)
    errs = []
    for name, t in (("got", got), ("want", want)):
        g = t.detach().to("cpu", torch.float64).numpy()[rows]
        errs.append(f"{name} max-abs vs oracle {float(np.nanmax(np.abs(g - ref))):.3e}")
    return (f"{label}: {len(differ)} token rows differ (sequences {seqs[:12]}, q_lens "
            f"{[int(cu[s + 1] - cu[s]) for s in seqs[:12]]}), {nan_rows} of them with NaN; " + ", ".join(errs))
