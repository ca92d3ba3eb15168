"""Float64 CPU oracle for MLA decoding over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may load this; the product path never does.  It
shares no code with the GPU sources.  The arithmetic lives in mla_oracle.c
(plain C, float64, OpenMP over query rows); this module compiles it with gcc and
marshals numpy arrays through ctypes.  See mla_oracle.c for the definition and
the passages of the FlashMLA pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

D_QK = 576
D_V = 512


def build(force: bool = True) -> str:
    """Compile mla_oracle.c with gcc into oracle/liboracle.so (IEEE float64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        L.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_token_bytes.restype = ctypes.c_int64
        L.oracle_token_bytes.argtypes = [ctypes.c_int]
        L.oracle_token_latent.restype = None
        L.oracle_token_latent.argtypes = [P, ctypes.c_int, P]
        L.oracle_attend.restype = None
        L.oracle_attend.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int64, ctypes.c_double, P, P]
        L.oracle_lse_combine.restype = None
        L.oracle_lse_combine.argtypes = [ctypes.c_int64, P, P, P, P]
        L.oracle_mla_decode.restype = None
        L.oracle_mla_decode.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, P,
                                        P, ctypes.c_int, ctypes.c_int, ctypes.c_double, P, ctypes.c_int64, P, P]
        L.oracle_fp8_dequant_bf16.restype = ctypes.c_uint16
        L.oracle_fp8_dequant_bf16.argtypes = [ctypes.c_uint8, ctypes.c_float]
        L.oracle_schedule.restype = ctypes.c_int
        L.oracle_schedule.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def bf16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16).reshape(-1)
    return np.array([lib().oracle_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def e4m3fn_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint8).reshape(-1)
    return np.array([lib().oracle_e4m3fn_to_f64(int(x)) for x in c], dtype=np.float64)


def token_bytes(is_fp8: bool) -> int:
    return int(lib().oracle_token_bytes(int(is_fp8)))


def token_latent(token: np.ndarray, is_fp8: bool) -> np.ndarray:
    t = _c(token, np.uint8).reshape(-1)
    if t.size != token_bytes(is_fp8):
        raise ValueError("token has %d bytes" % t.size)
    out = np.zeros(D_QK, dtype=np.float64)
    lib().oracle_token_latent(_ptr(t), int(is_fp8), _ptr(out))
    return out


def attend(q_row_bits, kvcache_bytes: np.ndarray, is_fp8: bool, block_table_row, positions,
           scale: float) -> Tuple[np.ndarray, float]:
    q = _c(q_row_bits, np.uint16).reshape(-1)
    kv = _c(kvcache_bytes, np.uint8)
    bt = _c(block_table_row, np.int32)
    pos = _c(positions, np.int64).reshape(-1)
    o = np.zeros(D_V, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib().oracle_attend(_ptr(q), _ptr(kv), int(is_fp8), _ptr(bt), _ptr(pos), int(pos.size), float(scale), _ptr(o),
                        _ptr(lse))
    return o, float(lse[0])


def lse_combine(o_parts, lse_parts) -> Tuple[np.ndarray, float]:
    op = _c(o_parts, np.float64).reshape(-1, D_V)
    lp = _c(lse_parts, np.float64).reshape(-1)
    o = np.zeros(D_V, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib().oracle_lse_combine(int(lp.size), _ptr(op), _ptr(lp), _ptr(o), _ptr(lse))
    return o, float(lse[0])


def mla_decode(q_bits, kvcache_bytes, is_fp8: bool, block_table, cache_seqlens, indices, scale: float,
               rows=None, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """o [n_rows, 512] and lse [n_rows] in float64 for the listed flat rows
    (b * s_q + s) * h_q + h, or all rows when rows is None.

    q_bits: uint16/int16 [B, s_q, h_q, 576]; kvcache_bytes: uint8 view of the
    cache; block_table int32 [B, max_blocks]; cache_seqlens int32 [B];
    indices int32 [B, s_q, topk] or None.  causal: dense only; query token s
    sees positions j <= seqlen_b - s_q + s.
    """
    q = _c(q_bits, np.uint16)
    if q.ndim != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be [B, s_q, h_q, 576]")
    B, s_q, h_q = q.shape[:3]
    kv = _c(kvcache_bytes, np.uint8)
    bt = _c(block_table, np.int32)
    sl = _c(cache_seqlens, np.int32)
    idx = None if indices is None else _c(indices, np.int32)
    topk = 0 if idx is None else int(idx.shape[2])
    if causal and idx is not None:
        raise ValueError("causal masking is defined for dense decoding only")
    if rows is None:
        r = None
        n = B * s_q * h_q
    else:
        r = _c(rows, np.int64).reshape(-1)
        n = int(r.size)
    o = np.zeros((n, D_V), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    lib().oracle_mla_decode(_ptr(q), B, s_q, h_q, _ptr(kv), int(is_fp8), _ptr(bt), int(bt.shape[1]), _ptr(sl), _ptr(idx),
                            topk, int(bool(causal)), float(scale), _ptr(r), n, _ptr(o), _ptr(lse))
    return o, lse


def problem_decode(prob, rows=None, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """mla_decode on an mla_inputs.Problem (CPU torch tensors)."""
    import torch

    q = prob.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kv = prob.kvcache.contiguous().view(torch.uint8).numpy()
    idx = None if prob.indices is None else prob.indices.numpy()
    return mla_decode(q, kv, prob.is_fp8, prob.block_table.numpy(), prob.cache_seqlens.numpy(), idx,
                      prob.softmax_scale, rows, causal)


def fp8_dequant_bf16(codes, scales) -> np.ndarray:
    """bf16 bits of bf16_RNE(fp32_RNE(e4m3(code) * scale)), elementwise."""
    c = _c(codes, np.uint8).reshape(-1)
    s = _c(scales, np.float32).reshape(-1)
    if s.size == 1:
        s = np.full(c.size, s[0], dtype=np.float32)
    L = lib()
    return np.array([L.oracle_fp8_dequant_bf16(int(a), float(b)) for a, b in zip(c, s)], dtype=np.uint16)


def schedule(cache_seqlens, s_q: int, topk: int, num_workers: int, min_tiles: int) -> Tuple[np.ndarray, np.ndarray]:
    """The split/tile schedule rule: (sched int32 [W, 8], split_offset int32 [n_streams + 1])."""
    sl = _c(cache_seqlens, np.int32)
    B = int(sl.size)
    n_streams = B * s_q if topk > 0 else B
    sched = np.zeros((num_workers, 8), dtype=np.int32)
    off = np.zeros(n_streams + 1, dtype=np.int32)
    lib().oracle_schedule(_ptr(sl), B, s_q, topk, num_workers, min_tiles, _ptr(sched), _ptr(off))
    return sched, off
