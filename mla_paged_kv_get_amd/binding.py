"""Python binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the decode runs in the library's HIP kernels.  The
functions carry the C names.  If the library is missing the binding raises; it
never falls back to another implementation.

torch is imported before the library is loaded so that the library binds to the
HIP runtime torch already loaded (same SONAME) and torch's stream handles are
valid for it.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")
_lib = None

MLA_OK = 0
ERRORS = {-1: "MLA_ERR_INVALID_ARG", -2: "MLA_ERR_UNSUPPORTED", -3: "MLA_ERR_BUFFER_TOO_SMALL", -4: "MLA_ERR_HIP"}
D_QK = 576
D_V = 512
PAGE = 64
FP8_TOKEN_BYTES = 656


class MlaError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__("%s failed with %s (%d): %s" % (where, ERRORS.get(code, "?"), code, msg))
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libmla_decode.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is missing; build it with `python -m mla_paged_kv_get_amd.build` "
                               "(or __graft_entry__.build())" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_last_error.argtypes = []
        L.mla_get_metadata_size.restype = I
        L.mla_get_metadata_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Z), ctypes.POINTER(Z), ctypes.POINTER(I)]
        L.mla_get_metadata.restype = I
        L.mla_get_metadata.argtypes = [P, I, I, I, I, I, I, I, P, Z, P]
        L.mla_decode_with_kvcache.restype = I
        L.mla_decode_with_kvcache.argtypes = [P, P, I64, P, I, P, I, I, I, I, I, I, ctypes.c_float, P, Z, I, P, I, I, I,
                                              P, Z, P, P, P]
        L.mla_decode_with_kvcache_noalloc.restype = I
        L.mla_decode_with_kvcache_noalloc.argtypes = [P, P, I64, P, I, P, I, I, I, I, I, I, ctypes.c_float, P, Z, I, P,
                                                      I, I, I, P, P, P]
        L.mla_sparse_prefill_workspace_size.restype = I
        L.mla_sparse_prefill_workspace_size.argtypes = [I, I, I, I64, I, I, ctypes.POINTER(Z), ctypes.POINTER(I)]
        L.mla_sparse_prefill.restype = I
        L.mla_sparse_prefill.argtypes = [P, P, I64, P, I, I, I, I, I, I, ctypes.c_float, I, P, Z, P, P, P]
        L.mla_debug_dequant_fp8.restype = I
        L.mla_debug_dequant_fp8.argtypes = [P, I64, P, P]
        L.mla_set_decode_kernel_events.restype = I
        L.mla_set_decode_kernel_events.argtypes = [P, P]
        L.mla_set_merge_mode.restype = I
        L.mla_set_merge_mode.argtypes = [I]
        _lib = L
    return _lib


MLA_MERGE_OFF, MLA_MERGE_ON = 0, 1


def mla_set_merge_mode(mode: int) -> None:
    """Where this thread's later decode calls merge split results: MLA_MERGE_OFF
    (default: the combine kernel) or MLA_MERGE_ON (in the decode kernel, by the
    last split of each row tile, when every stream provably has at most 4
    splits)."""
    _check(lib().mla_set_merge_mode(int(mode)), "mla_set_merge_mode")


def mla_last_error() -> str:
    return lib().mla_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != MLA_OK:
        raise MlaError(rc, where, mla_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mla_get_metadata_size(B: int, s_q: int, h_q: int, h_kv: int = 1, topk: int = 0,
                          num_workers: int = 0) -> Tuple[int, int, int]:
    """(metadata bytes, workspace bytes, workers used)."""
    mb, wb, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int()
    _check(lib().mla_get_metadata_size(B, s_q, h_q, h_kv, topk, num_workers, ctypes.byref(mb), ctypes.byref(wb),
                                       ctypes.byref(w)), "mla_get_metadata_size")
    return int(mb.value), int(wb.value), int(w.value)


@dataclass
class Metadata:
    """Schedule of one decode step; valid while the lengths and shape stay the same."""

    tensor: torch.Tensor  # int32, on the device
    num_workers: int
    workspace_bytes: int
    B: int
    s_q: int
    h_q: int
    h_kv: int
    topk: int
    is_fp8: bool

    def total_splits(self) -> int:
        """Number of (stream, KV range) splits in the schedule (synchronises)."""
        return int(self.tensor[5].item())


def mla_get_metadata(cache_seqlens: torch.Tensor, s_q: int, h_q: int, h_kv: int = 1, topk: int = 0,
                     is_fp8: bool = False, num_workers: int = 0, out: Optional[torch.Tensor] = None) -> Metadata:
    """Run the scheduler kernel for a decode step (B = len(cache_seqlens)); `out`
    optionally supplies the int32 device buffer to fill (at least the size call's
    metadata bytes)."""
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda or not cache_seqlens.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous int32 device tensor")
    B = int(cache_seqlens.numel())
    with torch.cuda.device(cache_seqlens.device):
        mb, wb, w = mla_get_metadata_size(B, s_q, h_q, h_kv, topk, num_workers)
        if out is not None:
            if out.dtype != torch.int32 or out.device != cache_seqlens.device or not out.is_contiguous() or \
                    out.numel() * 4 < mb:
                raise ValueError("out must be a contiguous int32 tensor of >= %d bytes on %s" % (mb, cache_seqlens.device))
            meta = out
        else:
            meta = torch.empty(mb // 4, dtype=torch.int32, device=cache_seqlens.device)
        _check(lib().mla_get_metadata(_ptr(cache_seqlens), B, s_q, h_q, h_kv, topk, int(is_fp8), w, _ptr(meta),
                                      meta.numel() * 4,
                                      _stream(cache_seqlens.device)), "mla_get_metadata")
    return Metadata(meta, w, wb, B, s_q, h_q, h_kv, topk, bool(is_fp8))


def mla_decode_with_kvcache(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor,
                            cache_seqlens: torch.Tensor, d_v: int, metadata: Metadata,
                            indices: Optional[torch.Tensor] = None, is_fp8: bool = False,
                            softmax_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None,
                            causal: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """o (bf16 [B, s_q, h_q, 512]) and lse (fp32 [B, s_q, h_q]) of MLA decode.

    q: bf16 [B, s_q, h_q, 576]; kvcache: bf16 [num_blocks, 64, (1,) 576] or uint8
    [num_blocks, 64, (1,) 656] with is_fp8; block_table int32 [B, max_blocks];
    cache_seqlens int32 [B]; indices int32 [B, s_q, topk] for sparse decode.
    causal (dense only): query token s of s_q sees cache positions
    <= seqlen - s_q + s.
    """
    dev = q.device
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be bf16 [B, s_q, h_q, 576]")
    B, s_q, h_q = (int(x) for x in q.shape[:3])
    for name, t in (("q", q), ("kvcache", kvcache), ("block_table", block_table), ("cache_seqlens", cache_seqlens)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be contiguous and on %s" % (name, dev))
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != B:
        raise ValueError("cache_seqlens must be int32 [B]")
    width = FP8_TOKEN_BYTES if is_fp8 else D_QK
    want = torch.uint8 if is_fp8 else torch.bfloat16
    if kvcache.dtype != want or kvcache.shape[-1] != width or kvcache.shape[1] != PAGE:
        raise ValueError("kvcache must be %s [num_blocks, 64, (1,) %d]" % (want, width))
    num_blocks = int(kvcache.shape[0])
    topk = 0
    if indices is not None:
        if indices.dtype != torch.int32 or indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q):
            raise ValueError("indices must be int32 [B, s_q, topk]")
        if indices.device != dev or not indices.is_contiguous():
            raise ValueError("indices must be contiguous and on %s" % dev)
        topk = int(indices.shape[2])
    m = metadata
    if (m.B, m.s_q, m.h_q, m.topk) != (B, s_q, h_q, topk):
        raise ValueError("metadata was built for another shape")
    if workspace is None:
        workspace = torch.empty(m.workspace_bytes, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(D_QK)
    with torch.cuda.device(dev):
        _check(lib().mla_decode_with_kvcache(
            _ptr(q), _ptr(kvcache), num_blocks, _ptr(block_table), int(block_table.shape[1]), _ptr(cache_seqlens), B,
            s_q, h_q, m.h_kv, D_QK, d_v, scale, _ptr(m.tensor), m.tensor.numel() * 4, m.num_workers, _ptr(indices),
            topk, int(is_fp8), int(bool(causal)), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _ptr(out), _ptr(lse), _stream(dev)), "mla_decode_with_kvcache")
    return out, lse


def mla_decode_with_kvcache_noalloc(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor,
                                    cache_seqlens: torch.Tensor, d_v: int, metadata: Metadata, out: torch.Tensor,
                                    lse: torch.Tensor, indices: Optional[torch.Tensor] = None, is_fp8: bool = False,
                                    softmax_scale: Optional[float] = None, causal: bool = False) -> None:
    """mla_decode_with_kvcache without a workspace argument: the library's static
    scratch holds the split workspace, and the caller passes o (bf16
    [B, s_q, h_q, 512]) and lse (fp32 [B, s_q, h_q]), so nothing is allocated."""
    dev = q.device
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be bf16 [B, s_q, h_q, 576]")
    B, s_q, h_q = (int(x) for x in q.shape[:3])
    for name, t in (("q", q), ("kvcache", kvcache), ("block_table", block_table), ("cache_seqlens", cache_seqlens),
                    ("out", out), ("lse", lse)) + ((("indices", indices),) if indices is not None else ()):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be contiguous and on %s" % (name, dev))
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, s_q, h_q, D_V):
        raise ValueError("out must be bf16 [B, s_q, h_q, 512]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, s_q, h_q):
        raise ValueError("lse must be fp32 [B, s_q, h_q]")
    topk = 0 if indices is None else int(indices.shape[2])
    m = metadata
    if (m.B, m.s_q, m.h_q, m.topk) != (B, s_q, h_q, topk):
        raise ValueError("metadata was built for another shape")
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(D_QK)
    with torch.cuda.device(dev):
        _check(lib().mla_decode_with_kvcache_noalloc(
            _ptr(q), _ptr(kvcache), int(kvcache.shape[0]), _ptr(block_table), int(block_table.shape[1]),
            _ptr(cache_seqlens), B, s_q, h_q, m.h_kv, D_QK, d_v, scale, _ptr(m.tensor), m.tensor.numel() * 4,
            m.num_workers, _ptr(indices), topk, int(is_fp8), int(bool(causal)), _ptr(out), _ptr(lse), _stream(dev)),
            "mla_decode_with_kvcache_noalloc")


def mla_sparse_prefill(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                       softmax_scale: Optional[float] = None, num_workers: int = 0,
                       workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """o (bf16 [s_q, h_q, 512]) and lse (fp32 [s_q, h_q]) of token-sparse prefill.

    q: bf16 [s_q, h_q, 576]; kv: bf16 [s_kv, (1,) 576], one contiguous sequence;
    indices: int32 [s_q, (1,) topk] of positions in [0, s_kv) or -1 (skipped).
    """
    dev = q.device
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != D_QK:
        raise ValueError("q must be bf16 [s_q, h_q, 576]")
    s_q, h_q = int(q.shape[0]), int(q.shape[1])
    if kv.dtype != torch.bfloat16 or kv.shape[-1] != D_QK or kv.numel() % D_QK:
        raise ValueError("kv must be bf16 [s_kv, (1,) 576]")
    s_kv = kv.numel() // D_QK
    if indices.dtype != torch.int32 or indices.shape[0] != s_q or indices.dim() not in (2, 3):
        raise ValueError("indices must be int32 [s_q, (1,) topk]")
    topk = int(indices.shape[-1])
    for name, t in (("q", q), ("kv", kv), ("indices", indices)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be contiguous and on %s" % (name, dev))
    need, W = ctypes.c_size_t(0), ctypes.c_int(0)
    with torch.cuda.device(dev):
        _check(lib().mla_sparse_prefill_workspace_size(s_q, h_q, 1, s_kv, topk, int(num_workers), ctypes.byref(need),
                                                       ctypes.byref(W)), "mla_sparse_prefill_workspace_size")
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=dev)
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(D_QK)
    with torch.cuda.device(dev):
        _check(lib().mla_sparse_prefill(
            _ptr(q), _ptr(kv), s_kv, _ptr(indices), s_q, h_q, 1, topk, D_QK, D_V, scale, int(num_workers),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev)),
            "mla_sparse_prefill")
    return out, lse


def mla_debug_dequant_fp8(tokens: torch.Tensor) -> torch.Tensor:
    """bf16 [n, 576] decode of uint8 [n, 656] FP8 tokens (test hook)."""
    if tokens.dtype != torch.uint8 or tokens.shape[-1] != FP8_TOKEN_BYTES or not tokens.is_contiguous():
        raise ValueError("tokens must be contiguous uint8 [..., 656]")
    n = tokens.numel() // FP8_TOKEN_BYTES
    out = torch.empty((n, D_QK), dtype=torch.bfloat16, device=tokens.device)
    with torch.cuda.device(tokens.device):
        _check(lib().mla_debug_dequant_fp8(_ptr(tokens), n, _ptr(out), _stream(tokens.device)), "mla_debug_dequant_fp8")
    return out


class DecodeKernelTimer:
    """Bench hook: HIP events around the split-KV decode kernel alone.

    Each call of `record(fn)` sets fresh start/stop events through
    mla_set_decode_kernel_events, runs fn() (which must make exactly one
    mla_decode_with_kvcache call on this thread) and clears the hook;
    `durations_ms()` synchronises and returns one duration per recorded call.
    The events come from the HIP runtime the library itself is bound to and
    are created without the system-scope fence (hipEventDisableSystemFence):
    they only time, and a default event's cache write-back and invalidation
    between the kernels of a step would slow the very work being timed.
    """

    _DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self):
        lib()  # torch's HIP runtime is loaded and shared with the library by now
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._pairs = []

    def _event(self):
        ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(ev), self._DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise MlaError(-4, "hipEventCreateWithFlags", "hipError_t %d" % rc)
        return ev

    def record(self, fn):
        a, b = self._event(), self._event()
        _check(lib().mla_set_decode_kernel_events(a, b), "mla_set_decode_kernel_events")
        try:
            fn()
        finally:
            lib().mla_set_decode_kernel_events(None, None)
        self._pairs.append((a, b))

    def durations_ms(self):
        out = []
        for a, b in self._pairs:
            rc = self._hip.hipEventSynchronize(b)
            if rc != 0:
                raise MlaError(-4, "hipEventSynchronize", "hipError_t %d" % rc)
            ms = ctypes.c_float()
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
            if rc != 0:
                raise MlaError(-4, "hipEventElapsedTime", "hipError_t %d" % rc)
            out.append(ms.value)
        for a, b in self._pairs:
            self._hip.hipEventDestroy(a)
            self._hip.hipEventDestroy(b)
        self._pairs = []
        return out
