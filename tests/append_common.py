"""Test helpers for the KV append: the step's new rows taken out of generated
pages.  Computed here from the page-table rows directly; neither the oracle nor
the GPU library is used."""
import numpy as np
import torch


def new_token_slots(inp):
    """Flat page-slot index (page * B + slot) of every new token, in token order,
    computed here from the page-table rows directly (vectorised per sequence)."""
    b = inp.k_pages.shape[1]
    cu, kv, table = inp.cu_q_lens.numpy(), inp.kv_lens.numpy(), inp.page_table.numpy()
    out = []
    for s in range(len(kv)):
        q_len = int(cu[s + 1] - cu[s])
        pos = np.arange(int(kv[s]) - q_len, int(kv[s]))
        out.append(table[s][pos // b].astype(np.int64) * b + pos % b)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def stale_pages_and_new_rows(inp, fill=float("nan")):
    """The step's new rows taken out of the generated pages (k_new, v_new in
    token order) and copies of the pages with those slots overwritten."""
    slots = new_token_slots(inp)
    p, b = inp.k_pages.shape[:2]
    out = []
    for pages in (inp.k_pages, inp.v_pages):
        flat = pages.reshape(p * b, *pages.shape[2:])
        new = flat[torch.from_numpy(slots)].clone()
        stale = pages.clone()
        stale.reshape(p * b, *pages.shape[2:])[torch.from_numpy(slots)] = fill
        out += [new, stale]
    return out   # k_new, k_stale, v_new, v_stale
