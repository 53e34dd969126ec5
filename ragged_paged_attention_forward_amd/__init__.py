"""Ragged paged attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``librpa.so`` (include/rpa.h): it only
checks and marshals arguments.  Every step of the attention runs in the HIP
kernels of the library; there is no fallback path.  PyTorch provides device
memory and the current stream.

    attn = RaggedPagedAttention(num_q_heads=8, num_kv_heads=1, head_dim=256,
                                page_size=128, max_num_seqs=512,
                                max_pages_per_seq=64, max_q_tokens=8192)
    out = attn.forward(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens,
                       window=0, scale=256 ** -0.5)
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import (RPA_ERR_HIP, RPA_ERR_INVALID_ARG, RPA_ERR_OOM, RPA_ERR_UNSUPPORTED,
                   RPA_KERNEL_APPEND, RPA_KERNEL_DECODE, RPA_KERNEL_MERGE, RPA_KERNEL_PREFILL,
                   RPA_KERNEL_STAGE, RPA_KERNEL_DECODE2, RPA_OK,
                   RPA_OPT_DECODE_MAX_ROWS, RPA_OPT_DECODE_SPLIT_KEYS, RPA_OPT_DECODE_WAVES,
                   RPA_OPT_FUSED_MERGE, RPA_OPT_KERNEL_TIMING, RPA_OPT_PATH, RPA_OPT_XCD_GROUPS,
                   RPA_OPT_PREFILL_SPLIT_KEYS, RPA_OPT_CONCURRENT, RPA_OPT_FP8_STAGE,
                   PlanInfo, RpaError, WorkItem)

__all__ = ["RaggedPagedAttention", "rpa_forward", "RpaError", "library_path", "RPA_OK",
           "RPA_ERR_INVALID_ARG", "RPA_ERR_UNSUPPORTED", "RPA_ERR_OOM", "RPA_ERR_HIP",
           "RPA_OPT_DECODE_SPLIT_KEYS", "RPA_OPT_PATH", "RPA_OPT_DECODE_MAX_ROWS",
           "RPA_OPT_DECODE_WAVES", "RPA_OPT_KERNEL_TIMING", "RPA_OPT_XCD_GROUPS", "RPA_OPT_FUSED_MERGE", "RPA_OPT_PREFILL_SPLIT_KEYS", "RPA_OPT_CONCURRENT", "RPA_OPT_FP8_STAGE", "RPA_KERNEL_PREFILL", "RPA_KERNEL_DECODE",
           "RPA_KERNEL_MERGE", "RPA_KERNEL_APPEND", "RPA_KERNEL_STAGE", "RPA_KERNEL_DECODE2", "KERNEL_KINDS", "probe_read", "probe_mfma",
           "probe_e4m3"]

KERNEL_KINDS = {"prefill": RPA_KERNEL_PREFILL, "decode": RPA_KERNEL_DECODE, "merge": RPA_KERNEL_MERGE,
                "append": RPA_KERNEL_APPEND, "stage": RPA_KERNEL_STAGE, "decode2": RPA_KERNEL_DECODE2}


def library_path() -> str:
    return _lib.LIB_PATH


def _host_i32(x) -> np.ndarray:
    if type(x) is np.ndarray and x.dtype == np.int32 and x.flags.c_contiguous:
        return x
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu")
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _host_addr(a: np.ndarray) -> int:
    """Address of a contiguous host array's first element (a.ctypes.data,
    which costs about a microsecond, only for arrays that cannot be viewed
    through ctypes directly: empty or read-only ones)."""
    try:
        return ctypes.addressof(ctypes.c_char.from_buffer(a))
    except (TypeError, ValueError, BufferError):
        return a.ctypes.data


# torch's current raw stream and device, without building Stream / device
# objects (each of those costs microseconds per call); the public calls where
# this build of torch lacks them
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream_handle(stream, device_index: int) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class RaggedPagedAttention:
    """One library context (fixed head counts, head size and page size)."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 max_num_seqs: int, max_pages_per_seq: int, max_q_tokens: int):
        self._lib = _lib.load()
        cfg = _lib.Config(num_q_heads, num_kv_heads, head_dim, page_size, max_num_seqs,
                          max_pages_per_seq, max_q_tokens)
        ctx = ctypes.c_void_p()
        st = self._lib.rpa_create(ctypes.byref(cfg), ctypes.byref(ctx))
        if st != RPA_OK:
            raise RpaError(st, f"rpa_create failed: {self._lib.rpa_status_string(st).decode()}")
        self._ctx = ctx
        self._timing_cap = 0
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.page_size = page_size
        self.max_pages_per_seq = max_pages_per_seq

    # -- lifetime -------------------------------------------------------------
    def close(self):
        if getattr(self, "_ctx", None) is not None and self._ctx.value:
            self._lib.rpa_destroy(self._ctx)
        self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def release_captured(self) -> None:
        """``rpa_release_captured``: no graph holding a captured call of this
        context will be replayed again; its pinned work lists become evictable."""
        st = self._lib.rpa_release_captured(self._ctx)
        if st != RPA_OK:
            raise self._error(st, "rpa_release_captured")

    def _error(self, st: int, what: str) -> RpaError:
        msg = self._lib.rpa_last_error(self._ctx).decode(errors="replace")
        return RpaError(st, f"{what}: {self._lib.rpa_status_string(st).decode()}: {msg}")

    # -- options / planner ----------------------------------------------------
    def set_option(self, option: int, value: int) -> None:
        st = self._lib.rpa_set_option(self._ctx, int(option), int(value))
        if st != RPA_OK:
            raise self._error(st, "rpa_set_option")
        if option == RPA_OPT_KERNEL_TIMING:
            self._timing_cap = int(value)

    def plan_info(self, cu_q_lens, kv_lens, window: int = 0) -> dict:
        """Build the work list on the host (``rpa_plan`` without copying items) and
        return its summary."""
        cu = _host_i32(cu_q_lens)
        kv = _host_i32(kv_lens)
        info = PlanInfo()
        st = self._lib.rpa_plan(self._ctx, _i32p(cu), _i32p(kv), int(kv.shape[0]), int(window),
                                ctypes.byref(info), None, 0)
        if st != RPA_OK:
            raise self._error(st, "rpa_plan")
        return info.as_dict()

    def plan(self, cu_q_lens, kv_lens, window: int = 0) -> Tuple[dict, list]:
        cu = _host_i32(cu_q_lens)
        kv = _host_i32(kv_lens)
        n = int(kv.shape[0])
        info = PlanInfo()
        st = self._lib.rpa_plan(self._ctx, _i32p(cu), _i32p(kv), n, int(window), ctypes.byref(info),
                                None, 0)
        if st != RPA_OK:
            raise self._error(st, "rpa_plan")
        total = info.num_prefill_items + info.num_decode_items
        items = (WorkItem * max(total, 1))()
        st = self._lib.rpa_plan(self._ctx, _i32p(cu), _i32p(kv), n, int(window), ctypes.byref(info),
                                items, total)
        if st != RPA_OK:
            raise self._error(st, "rpa_plan")
        return info.as_dict(), [items[i].as_dict() for i in range(total)]

    def kernel_times(self, kind: int) -> np.ndarray:
        """Per-launch durations (ms) recorded for a kernel kind since the last read.

        Recording is switched on with ``set_option(RPA_OPT_KERNEL_TIMING, n)``; this
        waits for the recorded launches to finish and clears their record."""
        buf = np.zeros(max(self._timing_cap, 1), np.float32)
        count = ctypes.c_int32(0)
        st = self._lib.rpa_kernel_times(self._ctx, int(kind),
                                        buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                        int(buf.shape[0]), ctypes.byref(count))
        if st != RPA_OK:
            raise self._error(st, "rpa_kernel_times")
        return buf[:min(count.value, buf.shape[0])].copy()

    # -- forward --------------------------------------------------------------
    def _checked(self, q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out, stream,
                 kv_dtype=torch.bfloat16):
        cu = _host_i32(cu_q_lens)
        kv = _host_i32(kv_lens)
        n = int(kv.shape[0])
        if cu.shape[0] != n + 1:
            raise ValueError("cu_q_lens must have num_seqs + 1 entries")
        if q.dtype != torch.bfloat16 or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous bf16 CUDA tensor")
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            if t.dtype != kv_dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {kv_dtype} CUDA tensor")
        if page_table.dtype != torch.int32 or not page_table.is_cuda or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 CUDA tensor")
        if q.dim() != 3 or q.shape[1] != self.num_q_heads or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [T, {self.num_q_heads}, {self.head_dim}]")
        if n and int(cu[-1]) != q.shape[0]:
            raise ValueError("q has a different token count than cu_q_lens[-1]")
        pool = (self.page_size, self.num_kv_heads, self.head_dim)
        if k_pages.dim() != 4 or tuple(k_pages.shape[1:]) != pool or k_pages.shape != v_pages.shape:
            raise ValueError(f"k_pages / v_pages must both be [P, {pool[0]}, {pool[1]}, {pool[2]}]")
        if page_table.dim() != 2 or page_table.shape[0] < n or page_table.shape[1] != self.max_pages_per_seq:
            raise ValueError(f"page_table must be [num_seqs, {self.max_pages_per_seq}]")
        if out is None:
            out = torch.empty_like(q)
        elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous bf16 tensor shaped like q")
        return cu, kv, n, out, _host_addr(cu), _host_addr(kv), _stream_handle(stream, q.get_device())

    def _call(self, fn, name, device_index: int, args):
        cur = _current_device() if _current_device is not None else torch.cuda.current_device()
        if device_index == cur:
            st = fn(*args)
        else:
            with torch.cuda.device(device_index):
                st = fn(*args)
        if st != RPA_OK:
            raise self._error(st, name)

    def forward(self, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                page_table: torch.Tensor, cu_q_lens, kv_lens, window: int = 0,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Enqueue one attention call on ``stream`` (default: torch's current stream)."""
        if scale is None:
            scale = float(self.head_dim) ** -0.5
        cu, kv, n, out, cu_p, kv_p, sp = self._checked(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out,
                                                        stream)
        self._call(self._lib.rpa_forward, "rpa_forward", q.get_device(),
                   (self._ctx, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), page_table.data_ptr(),
                    cu_p, kv_p, n, int(window), float(scale), out.data_ptr(), sp))
        return out

    def forward_noalloc(self, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                        page_table: torch.Tensor, cu_q_lens, kv_lens, window: int = 0,
                        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """``rpa_forward_noalloc``: the attention of ``forward`` without any device
        allocation by the library (its work list and partials go into the
        library's static scratch array).  ``out`` should be preallocated by
        callers that cannot allocate."""
        if scale is None:
            scale = float(self.head_dim) ** -0.5
        cu, kv, n, out, cu_p, kv_p, sp = self._checked(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out,
                                                        stream)
        self._call(self._lib.rpa_forward_noalloc, "rpa_forward_noalloc", q.get_device(),
                   (self._ctx, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), page_table.data_ptr(),
                    cu_p, kv_p, n, int(window), float(scale), out.data_ptr(), sp))
        return out

    def forward_append(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor, cu_q_lens,
                       kv_lens, window: int = 0, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Write the step's new K/V rows (``k_new`` / ``v_new``, [T, Hkv, D] bf16)
        into their page slots, then the attention of ``forward``, in one call."""
        if scale is None:
            scale = float(self.head_dim) ** -0.5
        cu, kv, n, out, cu_p, kv_p, sp = self._checked(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out,
                                                        stream)
        shape = (q.shape[0], self.num_kv_heads, self.head_dim)
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {list(shape)}")
        self._call(self._lib.rpa_forward_append, "rpa_forward_append", q.get_device(),
                   (self._ctx, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pages.data_ptr(),
                    v_pages.data_ptr(), page_table.data_ptr(), cu_p, kv_p, n, int(window),
                    float(scale), out.data_ptr(), sp))
        return out

    def forward_fp8(self, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                    k_scales: torch.Tensor, v_scales: torch.Tensor, page_table: torch.Tensor, cu_q_lens,
                    kv_lens, window: int = 0, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """``forward`` over an fp8 KV cache: ``k_pages`` / ``v_pages`` hold OCP
        FP8 E4M3 bytes (uint8, [P, page_size, Hkv, D]) and ``k_scales`` /
        ``v_scales`` one float32 per KV head (CUDA tensors); element bytes
        stand for their E4M3 value times their head's scale."""
        if scale is None:
            scale = float(self.head_dim) ** -0.5
        cu, kv, n, out, cu_p, kv_p, sp = self._checked(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out,
                                                        stream, kv_dtype=torch.uint8)
        for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
            if (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()
                    or tuple(t.shape) != (self.num_kv_heads,)):
                raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape [{self.num_kv_heads}]")
        self._call(self._lib.rpa_forward_fp8, "rpa_forward_fp8", q.get_device(),
                   (self._ctx, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), k_scales.data_ptr(),
                    v_scales.data_ptr(), page_table.data_ptr(), cu_p, kv_p, n, int(window),
                    float(scale), out.data_ptr(), sp))
        return out

    def forward_fp8_append(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                           k_pages: torch.Tensor, v_pages: torch.Tensor, k_scales: torch.Tensor,
                           v_scales: torch.Tensor, page_table: torch.Tensor, cu_q_lens, kv_lens, window: int = 0,
                           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Quantize the step's new K/V rows (bf16 ``[T, Hkv, D]``) into their
        slots of the fp8 pools, then the attention of ``forward_fp8``."""
        if scale is None:
            scale = float(self.head_dim) ** -0.5
        cu, kv, n, out, cu_p, kv_p, sp = self._checked(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, out,
                                                        stream, kv_dtype=torch.uint8)
        shape = (q.shape[0], self.num_kv_heads, self.head_dim)
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {list(shape)}")
        for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
            if (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()
                    or tuple(t.shape) != (self.num_kv_heads,)):
                raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape [{self.num_kv_heads}]")
        self._call(self._lib.rpa_forward_fp8_append, "rpa_forward_fp8_append", q.get_device(),
                   (self._ctx, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pages.data_ptr(),
                    v_pages.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(), page_table.data_ptr(),
                    cu_p, kv_p, n, int(window), float(scale), out.data_ptr(), sp))
        return out

    __call__ = forward


def rpa_forward(q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, window: int = 0,
                scale: Optional[float] = None, out=None):
    """One-shot call with a temporary context sized to the arguments."""
    kv = _host_i32(kv_lens)
    attn = RaggedPagedAttention(q.shape[1], k_pages.shape[2], q.shape[2], k_pages.shape[1],
                                max(1, kv.shape[0]), page_table.shape[1], max(1, q.shape[0]))
    try:
        res = attn.forward(q, k_pages, v_pages, page_table, cu_q_lens, kv, window, scale, out)
        torch.cuda.current_stream(q.device).synchronize()
        return res
    finally:
        attn.close()


def probe_read(src: torch.Tensor, nbytes: int, workgroups: int, sink: torch.Tensor,
               stream: Optional[torch.cuda.Stream] = None, threads: int = 256, loads_in_flight: int = 8) -> None:
    """Enqueue the streaming-read probe over the first ``nbytes`` of ``src``
    (``rpa_probe_read``); ``sink`` holds ``workgroups * threads`` int32."""
    if not src.is_cuda or not sink.is_cuda or sink.numel() * sink.element_size() < workgroups * threads * 4:
        raise ValueError("src and sink must be CUDA tensors; sink needs workgroups * threads words")
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds src")
    stream = stream or torch.cuda.current_stream(src.device)
    st = _lib.load().rpa_probe_read(src.data_ptr(), int(nbytes), int(workgroups), int(threads),
                                    int(loads_in_flight), sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
    if st != RPA_OK:
        raise RpaError(st, "rpa_probe_read")


def probe_mfma(workgroups: int, iterations: int, sink: torch.Tensor,
               stream: Optional[torch.cuda.Stream] = None) -> int:
    """Enqueue the MFMA-throughput probe (``rpa_probe_mfma``); returns its FLOP count."""
    if not sink.is_cuda or sink.numel() * sink.element_size() < workgroups * 512 * 4:
        raise ValueError("sink must be a CUDA tensor of workgroups * 512 floats")
    stream = stream or torch.cuda.current_stream(sink.device)
    st = _lib.load().rpa_probe_mfma(int(workgroups), int(iterations), sink.data_ptr(),
                                    ctypes.c_void_p(stream.cuda_stream))
    if st != RPA_OK:
        raise RpaError(st, "rpa_probe_mfma")
    return int(workgroups) * 8 * int(iterations) * 4 * 32768


def probe_e4m3(src: torch.Tensor, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 values of the E4M3 bytes ``src`` (uint8 CUDA tensor, size a
    multiple of 8), converted by the fp8 decode kernel's own conversion."""
    if src.dtype != torch.uint8 or not src.is_cuda or not src.is_contiguous() or src.numel() % 8:
        raise ValueError("src must be a contiguous uint8 CUDA tensor with a multiple of 8 elements")
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    lib = _lib.load()
    stream = torch.cuda.current_stream(src.device)
    st = lib.rpa_probe_e4m3(src.data_ptr(), dst.data_ptr(), src.numel(), ctypes.c_void_p(stream.cuda_stream))
    if st != RPA_OK:
        raise RpaError(st, "rpa_probe_e4m3")
    return dst
