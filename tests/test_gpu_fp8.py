"""GPU checks of rpa_forward_fp8 (through the C ABI): attention over a KV
cache held as OCP FP8 E4M3 bytes with per-KV-head K and V scales matches the
oracle's fp8 forward (max-abs <= 2e-2, mean-abs <= 2e-3, no NaN), and the
kernel's byte conversion matches torch's E4M3 decoding for every byte.  Page
slots past kv_len and the trap page hold the E4M3 NaN byte, so a kernel that
reads them shows it in its output."""
import numpy as np
import pytest
import torch

import oracle.rpa_oracle as ora
import rpa_workloads as wl
from gpu_common import compare, gpu_available, make_attn

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def mixed_small(window, seed=205, page_size=128):
    rng = np.random.default_rng(seed)
    kv = rng.integers(64, 1500, 64)
    chunks = [(300, 300), (150, 230), (70, 400), (33, 80)]
    return wl.Workload(f"mixed_small_w{window}", chunks + [(1, int(k)) for k in kv], 8, 1, 256, page_size,
                       window, seed, length_draw=(64, 1500, 64))


CASES = {
    "tiny": lambda: wl.tiny(),
    "decode": lambda: wl.decode(),
    "decode_pages16": lambda: wl.custom([(1, 64 + 37 * i) for i in range(40)], 8, 1, 256, 16, 0, seed=41),
    "swa_prefill_1100": lambda: wl.swa_prefill(tokens=1100),
    "global_prefill_300": lambda: wl.global_prefill(tokens=300),
    "mixed_small_w0": lambda: mixed_small(0),
    "mixed_small_w1024_pages16": lambda: mixed_small(1024, page_size=16),
    "gqa4_d128_chunks": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 32, 0, seed=42),
    "with_empty_sequences": lambda: wl.custom([(0, 50), (3, 70), (0, 1), (1, 300), (0, 0), (17, 17)], 8, 2, 256, 64,
                                              0, seed=43),
    "mha_d64_window": lambda: wl.custom([(9, 200), (1, 65), (64, 64)], 4, 4, 64, 16, 33, seed=44),
    # page sizes that are not a multiple of 16 keys (a page id per lane in the
    # decode kernel), of 4 (a prefill wave's rows at d 256 in one page), and
    # of 16 but not 32 (16-key decode runs, a prefill wave's rows at d 128)
    "decode_pages8": lambda: wl.custom([(1, 64 + 37 * i) for i in range(40)], 8, 1, 256, 8, 0, seed=46),
    "mixed_small_w1024_pages24": lambda: mixed_small(1024, page_size=24),
    "gqa4_d128_chunks_pages48": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 48, 0,
                                                  seed=49),
    "gqa4_d128_chunks_pages24": lambda: wl.custom([(40, 100), (1, 17), (129, 129), (3, 1000)], 16, 4, 128, 24, 0,
                                                  seed=50),
    "g16_d128": lambda: wl.custom([(5, 90), (1, 400)], 16, 1, 128, 64, 0, seed=45),
    "g32_d128_prefill_only": lambda: wl.custom([(5, 90), (33, 400), (1, 70)], 32, 1, 128, 64, 0, seed=47),
}


def run_fp8(f: wl.Fp8Inputs, attn=None, path=0, stage=2):
    d = f.to("cuda")
    b = f.base
    if attn is None:
        attn = make_attn(b.workload)
        attn.set_option(R.RPA_OPT_PATH, path)
        attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = attn.forward_fp8(d.base.q, d.k_pages, d.v_pages, d.k_scales, d.v_scales, d.base.page_table,
                           b.cu_q_lens, b.kv_lens, b.window, b.scale)
    torch.cuda.synchronize()
    return out


def oracle_fp8(f: wl.Fp8Inputs, rows=None):
    b = f.base
    return ora.forward_fp8_rows(b.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens,
                                b.kv_lens, b.window, b.scale, rows)


def test_e4m3_conversion_matches_torch_for_every_byte():
    rng = np.random.default_rng(7)
    codes = np.concatenate([np.arange(256), rng.integers(0, 256, 4096)]).astype(np.uint8)
    src = torch.from_numpy(codes)
    got = R.probe_e4m3(src.cuda())
    torch.cuda.synchronize()
    want = src.view(torch.float8_e4m3fn).to(torch.bfloat16)
    g, w = got.cpu().view(torch.int16), want.view(torch.int16)
    nan = torch.isnan(want)
    assert torch.equal(torch.isnan(got.cpu()), nan)
    assert torch.equal(g[~nan], w[~nan])


ROUTES = {"prefill_converts": (0, 0), "staged_prefill": (0, 1), "all_decode": (3, 2)}


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("name", list(CASES))
def test_fp8_parity(name, route):
    """prefill_converts: prefill sequences through the prefill kernel, which
    loads the E4M3 tiles and converts them in LDS, the rest through the
    decode kernel; staged_prefill: the same after a staging kernel has
    converted their pages into a bf16 pool; all_decode: every token through
    the decode kernel (G <= 16)."""
    path, stage = ROUTES[route]
    w = CASES[name]()
    print(f"fp8 parity {name} {route}: seqs={w.num_seqs} T={w.total_q} d={w.head_dim} B={w.page_size} "
          f"W={w.window}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    out = run_fp8(f, path=path, stage=stage)
    compare(out, oracle_fp8(f), label=name)


def tile_edge_rows(attn, f):
    """First and last token row of every prefill query tile of the call's plan."""
    b = f.base
    _, items = attn.plan(b.cu_q_lens, b.kv_lens, b.window)
    rows = []
    for it in items:
        if it["kind"] == 0:
            rows += [it["q_start"], it["q_start"] + it["q_count"] - 1]
    return rows


@pytest.mark.parametrize("stage", [0, 1])
@pytest.mark.parametrize("window", [0, 1024])
def test_fp8_mixed_full_size_sampled(window, stage):
    w = wl.mixed(window=window)
    print(f"fp8 mixed full size W={window} stage={stage}: T={w.total_q}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = run_fp8(f, attn)
    t_q = w.total_q
    rows = wl.sample_rows(t_q, 48, seed=window + 3, must=[0, 4095, 4096, t_q - 513, t_q - 1])
    compare(out, oracle_fp8(f, rows), rows=rows, label=f"mixed_w{window}")


@pytest.mark.parametrize("stage", [0, 1])
@pytest.mark.parametrize("name", ["swa_prefill", "global_prefill"])
def test_fp8_prefill_full_size_sampled(name, stage):
    """Full-size fp8 prefills, both prefill routes: a seeded sample plus the
    first and last row of every query tile."""
    w = wl.by_name(name)
    print(f"fp8 {name} full size stage={stage}: T={w.total_q} d={w.head_dim}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = run_fp8(f, attn)
    t_q = w.total_q
    rows = wl.sample_rows(t_q, 24, seed=11, must=[0, 127, 128, 1023, 1024, t_q - 1] + tile_edge_rows(attn, f))
    compare(out, oracle_fp8(f, rows), rows=rows, label=name)


@pytest.mark.parametrize("stage", [0, 1])
@pytest.mark.parametrize("window", [0, 1024])
def test_fp8_long_contexts_sampled(window, stage):
    """Decodes over 40K-key contexts and a 2048-token chunk on a 30K prefix
    (a prefill key range of 235 pages: the prefill kernel's page-id window
    of 64 pages is reloaded as its tiles move on), both prefill routes;
    sampled rows, every row of the chunk's first and last tile included."""
    seqs = [(1, 40_000), (2048, 30_000), (1, 129), (3, 17_001)]
    w = wl.custom(seqs, 8, 1, 256, 128, window, seed=73 + window)
    print(f"fp8 long contexts W={window} stage={stage}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = run_fp8(f, attn)
    t = w.total_q
    cu = f.base.cu_q_lens.tolist()
    must = [0, cu[1], cu[1] + 1, cu[2] - 1, cu[2], t - 1, t - 2, t - 3] + tile_edge_rows(attn, f)
    rows = wl.sample_rows(t, 24, w.seed, must)
    compare(out, oracle_fp8(f, rows), rows=rows, label=f"fp8 long w{window} stage {stage}")


@pytest.mark.parametrize("stage", [0, 1, 2])
def test_fp8_staging_kernel_runs_only_when_asked(stage):
    """The staging kernel (timed as its own kind) runs with RPA_OPT_FP8_STAGE
    = 1 and not with 0, where the prefill kernel reads the E4M3 pages itself;
    with 2 (the default) the head size decides (d = 64, 256: no staging); every
    route matches the oracle."""
    w = CASES["mixed_small_w0"]()
    f = wl.make_fp8_inputs(w, poison=True)
    attn = make_attn(w)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 4)
    attn.set_option(R.RPA_OPT_FP8_STAGE, stage)
    out = run_fp8(f, attn)
    assert len(attn.kernel_times(R.RPA_KERNEL_STAGE)) == (1 if stage == 1 else 0)   # d = 256
    assert len(attn.kernel_times(R.RPA_KERNEL_PREFILL)) == 1
    assert len(attn.kernel_times(R.RPA_KERNEL_DECODE)) == 1
    compare(out, oracle_fp8(f), label=f"stage {stage}")


def test_fp8_is_bitwise_reproducible():
    f = wl.make_fp8_inputs(mixed_small(0), poison=True)
    attn = make_attn(f.base.workload)
    a = run_fp8(f, attn).clone()
    b = run_fp8(f, attn)
    assert torch.equal(a, b)


def test_fp8_and_bf16_calls_alternate_on_one_context():
    """The cached plan of an fp8 call (every token in decode items) is not the
    bf16 one for the same metadata: alternating calls each get their own."""
    w = wl.custom([(40, 100), (1, 300), (70, 70)], 8, 2, 128, 32, 0, seed=46)
    f = wl.make_fp8_inputs(w, poison=True)
    b = f.base
    attn = make_attn(w)
    d = b.to("cuda")
    ref16 = ora.forward_inputs(b)
    ref8 = oracle_fp8(f)
    for _ in range(2):
        out16 = attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, b.cu_q_lens, b.kv_lens, b.window, b.scale)
        torch.cuda.synchronize()
        compare(out16, ref16, label="bf16")
        compare(run_fp8(f, attn), ref8, label="fp8")


def test_fp8_graph_of_layers_replays_bitwise():
    """Four layers of one fp8 mixed step (their own pools and scales, one work
    list and one staging pool) captured into one graph: every replay equals
    the eager calls bit for bit."""
    w = mixed_small(1024)
    layers = 4
    host = [wl.make_fp8_inputs(w, seed=w.seed + 7 * i, poison=True) for i in range(layers)]
    dev = [h.to("cuda") for h in host]
    cu, kv = host[0].base.cu_q_lens, host[0].base.kv_lens
    attn = make_attn(w)

    def call(d, out=None):
        return attn.forward_fp8(d.base.q, d.k_pages, d.v_pages, d.k_scales, d.v_scales, d.base.page_table, cu, kv,
                                w.window, w.scale, out=out)
    eager = [call(d).clone() for d in dev]
    torch.cuda.synchronize()
    outs = [torch.empty_like(d.base.q) for d in dev]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d, o in zip(dev, outs):
            call(d, o)
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"layer {i}"
    compare(eager[3], oracle_fp8(host[3]), label="layer 3")


APPEND_CASES = ["tiny", "decode", "decode_pages16", "mixed_small_w0", "gqa4_d128_chunks", "with_empty_sequences",
                "mha_d64_window", "g32_d128_prefill_only"]


@pytest.mark.parametrize("name", APPEND_CASES)
def test_fp8_append_then_attend(name):
    """rpa_forward_fp8_append: the new tokens' bf16 K/V rows (the bf16 pools'
    rows at their slots) are quantized into slots that start as the E4M3 NaN
    byte; every byte of both pools must equal the oracle's fp8 append, and the
    attention that follows must match the oracle on the oracle's pools."""
    from append_common import new_token_slots
    w = CASES[name]()
    print(f"fp8 append {name}", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    b = f.base
    flat = torch.from_numpy(new_token_slots(b))
    hd = (w.num_kv_heads, w.head_dim)
    k_new = b.k_pages.reshape(-1, *hd)[flat].contiguous()
    v_new = b.v_pages.reshape(-1, *hd)[flat].contiguous()
    k_stale, v_stale = f.k_pages.clone(), f.v_pages.clone()
    k_stale.reshape(-1, *hd)[flat] = wl.NAN_E4M3
    v_stale.reshape(-1, *hd)[flat] = wl.NAN_E4M3
    want_k, want_v = ora.append_kv_fp8(k_stale, v_stale, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens,
                                       b.kv_lens, k_new, v_new)
    d = b.to("cuda")
    kp, vp = k_stale.cuda(), v_stale.cuda()
    attn = make_attn(w)
    out = attn.forward_fp8_append(d.q, k_new.cuda(), v_new.cuda(), kp, vp, f.k_scales.cuda(), f.v_scales.cuda(),
                                  d.page_table, b.cu_q_lens, b.kv_lens, w.window, w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp.cpu().numpy(), want_k)
    np.testing.assert_array_equal(vp.cpu().numpy(), want_v)
    ref = ora.forward_fp8_rows(b.q, want_k, want_v, f.k_scales, f.v_scales, b.page_table, b.cu_q_lens, b.kv_lens,
                               w.window, w.scale)
    compare(out, ref, label=name)


def test_fp8_append_saturates_and_keeps_nan_inf_and_signed_zero():
    """The append kernel's special branches at scales that are not powers of
    two: new elements beyond +-448 x scale (stored as +-448), NaN (0x7f),
    +-Inf (saturated), -0 (0x80), values near the subnormal end, and ordinary
    values; every byte of both pools must equal the oracle's fp8 append."""
    from append_common import new_token_slots
    w = wl.custom([(3, 40), (1, 77), (20, 20), (0, 9), (5, 300)], 8, 2, 128, 16, 0, seed=48)
    print("fp8 append special values", flush=True)
    f = wl.make_fp8_inputs(w, poison=True)
    b = f.base
    ks = torch.tensor([0.0173, 2.71], dtype=torch.float32)
    vs = torch.tensor([0.333, 0.00291], dtype=torch.float32)
    rng = np.random.default_rng(49)
    t_q, hkv, d = b.q.shape[0], w.num_kv_heads, w.head_dim
    scale_kv = torch.stack([ks, vs])                       # [2, Hkv]
    x = rng.standard_normal((2, t_q, hkv, d)).astype(np.float32)
    x *= rng.choice([0.001, 1.0, 200.0, 2000.0], size=x.shape).astype(np.float32)   # subnormal .. saturating
    new = torch.from_numpy(x) * scale_kv.view(2, 1, hkv, 1)
    flat = new.view(-1)
    special = torch.tensor([float("nan"), float("inf"), float("-inf"), -0.0, 0.0, 1e30, -1e30], dtype=torch.float32)
    idx = torch.from_numpy(rng.choice(flat.numel(), size=700, replace=False))
    flat[idx] = special[torch.arange(700) % special.numel()]
    k_new, v_new = new[0].to(torch.bfloat16).contiguous(), new[1].to(torch.bfloat16).contiguous()
    assert torch.isnan(k_new).any() and torch.isinf(v_new).any()
    assert (k_new.float().abs() > 448 * ks.view(1, -1, 1)).sum() > 100
    flat_slots = torch.from_numpy(new_token_slots(b))
    k_stale, v_stale = f.k_pages.clone(), f.v_pages.clone()
    k_stale.reshape(-1, hkv, d)[flat_slots] = wl.NAN_E4M3
    v_stale.reshape(-1, hkv, d)[flat_slots] = wl.NAN_E4M3
    want_k, want_v = ora.append_kv_fp8(k_stale, v_stale, ks, vs, b.page_table, b.cu_q_lens, b.kv_lens, k_new, v_new)
    d_ = b.to("cuda")
    kp, vp = k_stale.cuda(), v_stale.cuda()
    attn = make_attn(w)
    attn.forward_fp8_append(d_.q, k_new.cuda(), v_new.cuda(), kp, vp, ks.cuda(), vs.cuda(), d_.page_table,
                            b.cu_q_lens, b.kv_lens, w.window, w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp.cpu().numpy(), want_k)
    np.testing.assert_array_equal(vp.cpu().numpy(), want_v)
    got = kp.cpu().reshape(-1, hkv, d)[flat_slots]
    assert (got == 0x7E).any() and (got == 0xFE).any() and (got == 0x7F).any() and (got == 0x80).any()
