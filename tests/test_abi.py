"""C ABI checks that need no GPU: the library loads, exports every function
include/rpa.h declares, and rejects every invalid argument on the host before
anything is enqueued (no device call is reached in these tests)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from ragged_paged_attention_forward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rpa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rpa_create", "rpa_forward", "rpa_destroy", "rpa_status_string", "rpa_plan",
              "rpa_kernel_times"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for n in declared_functions():
        assert n in exported, n


def _ctx(hq=8, hkv=1, d=256, b=128, max_seqs=8, max_pages=8, max_q=64):
    lib = _lib.load()
    cfg = _lib.Config(hq, hkv, d, b, max_seqs, max_pages, max_q)
    ctx = ctypes.c_void_p()
    st = lib.rpa_create(ctypes.byref(cfg), ctypes.byref(ctx))
    return lib, st, ctx


def i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def test_create_rejects_bad_configs():
    assert _ctx(hq=6, hkv=4)[1] == _lib.RPA_ERR_INVALID_ARG
    assert _ctx(hkv=0)[1] == _lib.RPA_ERR_INVALID_ARG
    assert _ctx(b=0)[1] == _lib.RPA_ERR_INVALID_ARG
    assert _ctx(max_pages=0)[1] == _lib.RPA_ERR_INVALID_ARG
    assert _ctx(d=96)[1] == _lib.RPA_ERR_UNSUPPORTED
    assert _ctx(d=384)[1] == _lib.RPA_ERR_UNSUPPORTED
    lib = _lib.load()
    assert lib.rpa_create(None, None) == _lib.RPA_ERR_INVALID_ARG
    for d in (64, 128, 256, 512):
        lib, st, ctx = _ctx(d=d)
        assert st == _lib.RPA_OK
        lib.rpa_destroy(ctx)
    lib.rpa_destroy(None)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails on the host first


@pytest.mark.parametrize("case,cu,kv,n,window,scale,msg", [
    ("q_len > kv_len", [0, 5], [4], 1, 0, 1.0, "exceeds kv_len"),
    ("cu[0] != 0", [1, 5], [9], 1, 0, 1.0, "must be 0"),
    ("cu decreasing", [0, 5, 3], [9, 9], 2, 0, 1.0, "decreases"),
    ("negative kv_len", [0, 0], [-1], 1, 0, 1.0, "negative"),
    ("too many pages", [0, 1], [128 * 8 + 1], 1, 0, 1.0, "pages"),
    ("negative window", [0, 1], [5], 1, -3, 1.0, "window"),
    ("too many seqs", [0] * 10, [1] * 9, 9, 0, 1.0, "num_seqs"),
    ("negative seqs", [0], [], -1, 0, 1.0, "num_seqs"),
    ("too many tokens", [0, 65], [100], 1, 0, 1.0, "max_q_tokens"),
    ("nan scale", [0, 1], [5], 1, 0, float("nan"), "scale"),
    ("inf scale", [0, 1], [5], 1, 0, float("inf"), "scale"),
    ("zero scale", [0, 1], [5], 1, 0, 0.0, "scale"),
    ("negative scale", [0, 1], [5], 1, 0, -0.5, "scale"),
])
def test_forward_rejects_invalid_metadata(case, cu, kv, n, window, scale, msg):
    lib, st, ctx = _ctx()
    assert st == _lib.RPA_OK
    cu_a, cu_p = i32(cu)
    kv_a, kv_p = i32(kv if kv else [0])
    st = lib.rpa_forward(ctx, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, n, window, scale, ctypes.c_void_p(0x9000), None)
    assert st == _lib.RPA_ERR_INVALID_ARG, case
    assert msg in lib.rpa_last_error(ctx).decode(), lib.rpa_last_error(ctx)
    lib.rpa_destroy(ctx)


def test_forward_rejects_null_and_aliasing_pointers():
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 2])
    kv_a, kv_p = i32([7])
    for args in ((None, FAKE, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE, FAKE),
                 (FAKE, FAKE, None, FAKE, FAKE), (FAKE, FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, FAKE, None)):
        q, k, v, pt, out = args
        st = lib.rpa_forward(ctx, q, k, v, pt, cu_p, kv_p, 1, 0, 1.0, out, None)
        assert st == _lib.RPA_ERR_INVALID_ARG
    # out overlapping q
    st = lib.rpa_forward(ctx, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, ctypes.c_void_p(0x1000 + 64), None)
    assert st == _lib.RPA_ERR_INVALID_ARG and "overlaps" in lib.rpa_last_error(ctx).decode()
    # null metadata
    assert lib.rpa_forward(ctx, FAKE, FAKE, FAKE, FAKE, None, kv_p, 1, 0, 1.0, FAKE, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_forward(None, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, FAKE, None) == _lib.RPA_ERR_INVALID_ARG
    lib.rpa_destroy(ctx)


@pytest.mark.parametrize("case,cu,kv,n,window,scale,msg", [
    ("q_len > kv_len", [0, 5], [4], 1, 0, 1.0, "exceeds kv_len"),
    ("cu decreasing", [0, 5, 3], [9, 9], 2, 0, 1.0, "decreases"),
    ("too many pages", [0, 1], [128 * 8 + 1], 1, 0, 1.0, "pages"),
    ("negative window", [0, 1], [5], 1, -3, 1.0, "window"),
    ("too many tokens", [0, 65], [100], 1, 0, 1.0, "max_q_tokens"),
    ("zero scale", [0, 1], [5], 1, 0, 0.0, "scale"),
])
def test_forward_noalloc_rejects_invalid_arguments_before_any_device_call(case, cu, kv, n, window, scale, msg):
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32(cu)
    kv_a, kv_p = i32(kv)
    st = lib.rpa_forward_noalloc(ctx, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, n, window, scale,
                                 ctypes.c_void_p(0x9000), None)
    assert st == _lib.RPA_ERR_INVALID_ARG, case
    assert msg in lib.rpa_last_error(ctx).decode(), lib.rpa_last_error(ctx)
    cu_a, cu_p = i32([0, 2])
    kv_a, kv_p = i32([7])
    assert lib.rpa_forward_noalloc(ctx, FAKE, None, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, FAKE, None) == \
        _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_forward_noalloc(ctx, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, ctypes.c_void_p(0x1000 + 64),
                                   None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_forward_noalloc(None, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, FAKE, None) == \
        _lib.RPA_ERR_INVALID_ARG
    cu0_a, cu0_p = i32([0, 0])
    kv0_a, kv0_p = i32([3])   # no query tokens: nothing to do, no device call
    assert lib.rpa_forward_noalloc(ctx, None, None, None, None, cu0_p, kv0_p, 1, 0, 1.0, None, None) == _lib.RPA_OK
    lib.rpa_destroy(ctx)


def test_empty_call_returns_ok_without_device_work():
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 0, 0])
    kv_a, kv_p = i32([3, 0])
    # all-empty query batch: nothing to do, no device pointer is touched
    assert lib.rpa_forward(ctx, None, None, None, None, cu_p, kv_p, 2, 0, 1.0, None, None) == _lib.RPA_OK
    cu0, cu0_p = i32([0])
    assert lib.rpa_forward(ctx, None, None, None, None, cu0_p, None, 0, 0, 1.0, None, None) == _lib.RPA_OK
    lib.rpa_destroy(ctx)


def test_set_option_validation():
    lib, st, ctx = _ctx()
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PATH, 4) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PATH, 3) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_WAVES, 6) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_WAVES, 8) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_MAX_ROWS, 33) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_MAX_ROWS, -1) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_MAX_ROWS, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_MAX_ROWS, 17) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_DECODE_SPLIT_KEYS, -5) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, 999, 0) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PATH, 1) == _lib.RPA_OK
    assert lib.rpa_set_option(None, _lib.RPA_OPT_PATH, 1) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_KERNEL_TIMING, -1) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_KERNEL_TIMING, 65537) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_KERNEL_TIMING, 16) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_KERNEL_TIMING, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_CONCURRENT, 2) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_CONCURRENT, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_CONCURRENT, 1) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FP8_STAGE, 3) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FP8_STAGE, 2) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FP8_STAGE, -1) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FP8_STAGE, 1) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FP8_STAGE, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PREFILL_SPLIT_KEYS, -2) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PREFILL_SPLIT_KEYS, (1 << 30) + 1) == _lib.RPA_ERR_INVALID_ARG
    for v in (-1, 0, 512, 1 << 30):
        assert lib.rpa_set_option(ctx, _lib.RPA_OPT_PREFILL_SPLIT_KEYS, v) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_XCD_GROUPS, -1) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_XCD_GROUPS, 65) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_XCD_GROUPS, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_XCD_GROUPS, 8) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FUSED_MERGE, 2) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FUSED_MERGE, 0) == _lib.RPA_OK
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_FUSED_MERGE, 1) == _lib.RPA_OK
    lib.rpa_destroy(ctx)


def test_kernel_times_validation_and_empty_read():
    lib, st, ctx = _ctx()
    count = ctypes.c_int32(-7)
    buf = (ctypes.c_float * 4)()
    assert lib.rpa_kernel_times(None, 0, buf, 4, ctypes.byref(count)) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_kernel_times(ctx, 6, buf, 4, ctypes.byref(count)) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_kernel_times(ctx, -1, buf, 4, ctypes.byref(count)) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_kernel_times(ctx, 0, buf, -1, ctypes.byref(count)) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_kernel_times(ctx, 0, None, 4, ctypes.byref(count)) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_kernel_times(ctx, 0, buf, 4, None) == _lib.RPA_ERR_INVALID_ARG
    # nothing recorded yet: count 0, no device call
    assert lib.rpa_set_option(ctx, _lib.RPA_OPT_KERNEL_TIMING, 4) == _lib.RPA_OK
    for kind in (_lib.RPA_KERNEL_PREFILL, _lib.RPA_KERNEL_DECODE, _lib.RPA_KERNEL_MERGE, _lib.RPA_KERNEL_APPEND,
                 _lib.RPA_KERNEL_STAGE):
        assert lib.rpa_kernel_times(ctx, kind, buf, 4, ctypes.byref(count)) == _lib.RPA_OK
        assert count.value == 0
    assert lib.rpa_kernel_times(ctx, 1, None, 0, ctypes.byref(count)) == _lib.RPA_OK
    lib.rpa_destroy(ctx)


def test_status_strings():
    lib = _lib.load()
    for code, name in ((0, b"RPA_OK"), (-1, b"RPA_ERR_INVALID_ARG"), (-2, b"RPA_ERR_UNSUPPORTED"),
                       (-3, b"RPA_ERR_OOM"), (-4, b"RPA_ERR_HIP"), (7, b"RPA_ERR_UNKNOWN")):
        assert lib.rpa_status_string(code) == name


def test_probes_reject_bad_arguments_before_launch():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(64)
    addr = ctypes.addressof(buf)
    assert lib.rpa_probe_read(None, 64, 1, 256, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 64, 1, 256, 8, None, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 0, 1, 256, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 24, 1, 256, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 64, 0, 256, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 64, 65537, 256, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_read(addr, 64, 1, 128, 8, addr, None) == _lib.RPA_ERR_INVALID_ARG   # no such shape
    assert lib.rpa_probe_read(addr, 64, 1, 1024, 32, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_mfma(0, 1, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_mfma(1, 0, addr, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_mfma(1, 1, None, None) == _lib.RPA_ERR_INVALID_ARG


def test_forward_append_rejects_bad_pointers_before_launch():
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 2])
    kv_a, kv_p = i32([7])
    other = ctypes.c_void_p(0x900000)
    # q, k_new, v_new, k_pages, v_pages, page_table, out
    for args in ((FAKE, None, FAKE, FAKE, other, FAKE, other), (FAKE, FAKE, None, FAKE, other, FAKE, other),
                 (None, FAKE, FAKE, FAKE, other, FAKE, other), (FAKE, FAKE, FAKE, None, other, FAKE, other),
                 (FAKE, FAKE, FAKE, FAKE, other, None, other), (FAKE, FAKE, FAKE, FAKE, other, FAKE, None)):
        q, kn, vn, kp, vp, pt, out = args
        st = lib.rpa_forward_append(ctx, q, kn, vn, kp, vp, pt, cu_p, kv_p, 1, 0, 1.0, out, None)
        assert st == _lib.RPA_ERR_INVALID_ARG, args
    # the same buffer for keys and values
    st = lib.rpa_forward_append(ctx, FAKE, FAKE, FAKE, other, other, FAKE, cu_p, kv_p, 1, 0, 1.0,
                                ctypes.c_void_p(0x7000000), None)
    assert st == _lib.RPA_ERR_INVALID_ARG and "same buffer" in lib.rpa_last_error(ctx).decode()
    # metadata checks as for rpa_forward
    bad_kv_a, bad_kv_p = i32([1])   # q_len 2 > kv_len 1
    st = lib.rpa_forward_append(ctx, FAKE, FAKE, FAKE, FAKE, other, FAKE, cu_p, bad_kv_p, 1, 0, 1.0, other, None)
    assert st == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_forward_append(None, FAKE, FAKE, FAKE, FAKE, other, FAKE, cu_p, kv_p, 1, 0, 1.0, other,
                                  None) == _lib.RPA_ERR_INVALID_ARG
    lib.rpa_destroy(ctx)


def test_forward_fp8_rejects_bad_arguments_before_launch():
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 2])
    kv_a, kv_p = i32([7])
    other = ctypes.c_void_p(0x900000)
    # q, k_pages, v_pages, k_scales, v_scales, page_table, out
    for args in ((FAKE, FAKE, FAKE, None, FAKE, FAKE, other), (FAKE, FAKE, FAKE, FAKE, None, FAKE, other),
                 (None, FAKE, FAKE, FAKE, FAKE, FAKE, other), (FAKE, None, FAKE, FAKE, FAKE, FAKE, other),
                 (FAKE, FAKE, FAKE, FAKE, FAKE, None, other), (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)):
        q, kp, vp, ks, vs, pt, out = args
        st = lib.rpa_forward_fp8(ctx, q, kp, vp, ks, vs, pt, cu_p, kv_p, 1, 0, 1.0, out, None)
        assert st == _lib.RPA_ERR_INVALID_ARG, args
    bad_kv_a, bad_kv_p = i32([1])   # q_len 2 > kv_len 1
    st = lib.rpa_forward_fp8(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cu_p, bad_kv_p, 1, 0, 1.0, other, None)
    assert st == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_forward_fp8(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0, other,
                               None) == _lib.RPA_ERR_INVALID_ARG
    lib.rpa_destroy(ctx)


def test_probe_e4m3_rejects_bad_arguments():
    lib = _lib.load()
    addr = ctypes.c_void_p(0x800000)
    assert lib.rpa_probe_e4m3(None, addr, 64, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_e4m3(addr, None, 64, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_e4m3(addr, addr, 0, None) == _lib.RPA_ERR_INVALID_ARG
    assert lib.rpa_probe_e4m3(addr, addr, 12, None) == _lib.RPA_ERR_INVALID_ARG


def test_forward_fp8_append_rejects_bad_arguments_before_launch():
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 2])
    kv_a, kv_p = i32([7])
    other = ctypes.c_void_p(0x900000)
    # q, k_new, v_new, k_pages, v_pages, k_scales, v_scales, page_table, out
    for args in ((FAKE, None, FAKE, FAKE, other, FAKE, FAKE, FAKE, other),
                 (FAKE, FAKE, None, FAKE, other, FAKE, FAKE, FAKE, other),
                 (FAKE, FAKE, FAKE, FAKE, other, None, FAKE, FAKE, other),
                 (FAKE, FAKE, FAKE, FAKE, other, FAKE, None, FAKE, other),
                 (None, FAKE, FAKE, FAKE, other, FAKE, FAKE, FAKE, other),
                 (FAKE, FAKE, FAKE, FAKE, other, FAKE, FAKE, None, other)):
        q, kn, vn, kp, vp, ks, vs, pt, out = args
        st = lib.rpa_forward_fp8_append(ctx, q, kn, vn, kp, vp, ks, vs, pt, cu_p, kv_p, 1, 0, 1.0, out, None)
        assert st == _lib.RPA_ERR_INVALID_ARG, args
    st = lib.rpa_forward_fp8_append(ctx, FAKE, FAKE, FAKE, other, other, FAKE, FAKE, FAKE, cu_p, kv_p, 1, 0, 1.0,
                                    ctypes.c_void_p(0x7000000), None)
    assert st == _lib.RPA_ERR_INVALID_ARG and "same buffer" in lib.rpa_last_error(ctx).decode()
    lib.rpa_destroy(ctx)


def test_calls_without_query_tokens_accept_null_device_pointers():
    """A call whose sequences have no query tokens enqueues nothing and needs
    no device buffer (torch hands NULL for empty tensors), appending calls
    included; metadata is still checked."""
    lib, st, ctx = _ctx()
    cu_a, cu_p = i32([0, 0, 0])
    kv_a, kv_p = i32([5, 9])
    assert lib.rpa_forward(ctx, None, None, None, None, cu_p, kv_p, 2, 0, 1.0, None, None) == _lib.RPA_OK
    assert lib.rpa_forward_append(ctx, None, None, None, None, None, None, cu_p, kv_p, 2, 0, 1.0, None,
                                  None) == _lib.RPA_OK
    assert lib.rpa_forward_fp8(ctx, None, None, None, FAKE, FAKE, None, cu_p, kv_p, 2, 0, 1.0, None,
                               None) == _lib.RPA_OK
    assert lib.rpa_forward_fp8_append(ctx, None, None, None, None, None, FAKE, FAKE, None, cu_p, kv_p, 2, 0, 1.0,
                                      None, None) == _lib.RPA_OK
    bad_cu_a, bad_cu_p = i32([0, 0, -1])   # not non-decreasing
    assert lib.rpa_forward_append(ctx, None, None, None, None, None, None, bad_cu_p, kv_p, 2, 0, 1.0, None,
                                  None) == _lib.RPA_ERR_INVALID_ARG
    lib.rpa_destroy(ctx)
