"""The C-ABI library on the CPU: it loads, exports every declared entry point, and
its host-side validation rejects bad calls before touching a device.  No compute
call is made here (num_workers is always given, so no device query happens)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    """A private handle on the library (its prototypes do not touch the binding's)."""
    import torch  # noqa: F401  (binds the library to torch's HIP runtime, as in use)
    from mla_paged_kv_get_amd import binding

    binding.lib()
    h = ctypes.CDLL(binding.LIB_PATH)
    h.mla_last_error.restype = ctypes.c_char_p
    return h


def test_header_declares_the_boundary():
    syms = declared_symbols()
    assert set(syms) == {"mla_get_metadata_size", "mla_get_metadata", "mla_decode_with_kvcache", "mla_last_error",
                         "mla_debug_dequant_fp8", "mla_set_decode_kernel_events",
                         "mla_sparse_prefill_workspace_size", "mla_sparse_prefill",
                         "mla_decode_with_kvcache_noalloc", "mla_set_merge_mode"}


def test_library_exports_every_declared_symbol(L):
    for s in declared_symbols():
        assert hasattr(L, s), s


def test_library_is_gfx950_only():
    from mla_paged_kv_get_amd import binding

    data = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    assert b"gfx942" not in data and b"gfx90a" not in data


def sizes(L, B, s_q, h_q, h_kv=1, topk=0, W=256):
    mb, wb, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int()
    rc = L.mla_get_metadata_size(B, s_q, h_q, h_kv, topk, W, ctypes.byref(mb), ctypes.byref(wb), ctypes.byref(w))
    return rc, mb.value, wb.value, w.value


def test_metadata_and_workspace_sizes(L):
    # dense: B streams of s_q*h_q rows; sparse: B*s_q streams of h_q rows
    rc, mb, wb, w = sizes(L, 64, 1, 128, W=128)
    assert rc == 0 and w == 128
    n_streams, R = 64, 128
    # header, 8 words per worker, split offsets and tile starts, one arrival
    # counter per (stream, 64-row tile)
    assert mb == 4 * (16 + 8 * 128 + 2 * (n_streams + 1) + n_streams * 2)
    splits = 128 + n_streams
    part_o = -(-splits * R * 512 * 4 // 256) * 256
    assert wb == part_o + (-(-splits * R * 4 // 256) * 256)
    rc, mb, wb, w = sizes(L, 8, 2, 64, topk=2048, W=256)
    assert rc == 0
    assert mb == 4 * (16 + 8 * 256 + 2 * (16 + 1) + 16 * 1)
    rc, mb, wb, w = sizes(L, 3, 65, 2, W=16)  # 130 rows per stream: 3 row tiles
    assert rc == 0 and mb == 4 * (16 + 8 * 16 + 2 * (3 + 1) + 3 * 3)


def test_merge_mode_values(L):
    L.mla_set_merge_mode.argtypes = [ctypes.c_int]
    assert L.mla_set_merge_mode(2) == -1 and "merge mode" in L.mla_last_error().decode()
    assert L.mla_set_merge_mode(-1) == -1
    for m in (1, 0):  # ends on the default (off)
        assert L.mla_set_merge_mode(m) == 0


def test_size_call_rejects_bad_shapes(L):
    assert sizes(L, 0, 1, 16)[0] == -1
    assert sizes(L, 1, 1, 16, h_kv=2)[0] == -2
    assert "h_kv" in L.mla_last_error().decode()
    assert sizes(L, 1, 1, 16, topk=-1)[0] == -1
    assert sizes(L, 1, 1, 16, W=-3)[0] == -1


def decode(L, **kw):
    a = dict(q=0x1000, kv=0x2000, num_blocks=4, bt=0x3000, max_blocks=4, sl=0x4000, B=2, s_q=1, h_q=16, h_kv=1,
             d_qk=576, d_v=512, scale=0.0, meta=0x5000, meta_bytes=1 << 20, W=8, idx=None, topk=0, is_fp8=0,
             causal=0, ws=0x6000, ws_bytes=1 << 30, o=0x7000, lse=0x8000, stream=None)
    a.update(kw)
    L.mla_decode_with_kvcache.argtypes = None  # plain ints/None below
    f = L.mla_decode_with_kvcache
    P = ctypes.c_void_p
    return f(P(a["q"]), P(a["kv"]), ctypes.c_int64(a["num_blocks"]), P(a["bt"]), a["max_blocks"], P(a["sl"]), a["B"],
             a["s_q"], a["h_q"], a["h_kv"], a["d_qk"], a["d_v"], ctypes.c_float(a["scale"]), P(a["meta"]),
             ctypes.c_size_t(a["meta_bytes"]), a["W"], P(a["idx"]), a["topk"], a["is_fp8"], a["causal"], P(a["ws"]),
             ctypes.c_size_t(a["ws_bytes"]), P(a["o"]), P(a["lse"]), P(a["stream"]))


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=None), -1, "null"),
    (dict(d_qk=512), -2, "d_qk"),
    (dict(d_v=576), -2, "d_v"),
    (dict(h_kv=2), -2, "h_kv"),
    (dict(topk=8), -1, "indices"),
    (dict(idx=0x9000), -1, "indices"),
    (dict(is_fp8=2), -1, "is_fp8"),
    (dict(causal=2), -1, "causal"),
    (dict(causal=1, topk=8, idx=0x9000), -1, "causal"),
    (dict(q=0x1008), -1, "aligned"),
    (dict(meta_bytes=16), -3, "metadata"),
    (dict(ws_bytes=1024), -3, "workspace"),
    (dict(num_blocks=0), -1, "num_blocks"),
])
def test_decode_rejects_bad_calls_before_launching(L, kw, code, text):
    assert decode(L, **kw) == code
    assert text in L.mla_last_error().decode()


def test_debug_dequant_rejects_bad_calls(L):
    f = L.mla_debug_dequant_fp8
    f.argtypes = None
    assert f(None, ctypes.c_int64(1), ctypes.c_void_p(0x1000), None) == -1
    assert f(ctypes.c_void_p(0x1000), ctypes.c_int64(-1), ctypes.c_void_p(0x2000), None) == -1
    assert f(ctypes.c_void_p(0x1000), ctypes.c_int64(0), ctypes.c_void_p(0x2000), None) == 0  # nothing to do


def test_decode_kernel_events_hook_needs_both_or_neither(L):
    f = L.mla_set_decode_kernel_events
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert f(ctypes.c_void_p(0x1000), None) == -1
    assert "both" in L.mla_last_error().decode()
    assert f(None, ctypes.c_void_p(0x1000)) == -1
    assert f(None, None) == 0  # clearing is always fine (no HIP call is made)


def prefill_size(L, s_q, h_q, s_kv, topk, W=64, h_kv=1):
    L.mla_sparse_prefill_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                    ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t),
                                                    ctypes.POINTER(ctypes.c_int)]
    wb, w = ctypes.c_size_t(0), ctypes.c_int(0)
    rc = L.mla_sparse_prefill_workspace_size(s_q, h_q, h_kv, s_kv, topk, W, ctypes.byref(wb), ctypes.byref(w))
    return rc, wb.value, w.value


def test_sparse_prefill_workspace_size(L):
    """The prefill workspace holds the sequence length, one page-table entry per
    64 tokens, the schedule of s_q streams and the sparse decode workspace, in
    256-byte aligned parts; bad shapes are refused before anything runs."""
    rc, wb, w = prefill_size(L, 4096, 128, 8192, 2048, W=128)
    assert rc == 0 and w == 128
    rc_m, mb, dwb, _ = sizes(L, 1, 4096, 128, topk=2048, W=128)
    assert rc_m == 0
    pages = -(-8192 // 64) * 4
    assert wb == 256 + -(-pages // 256) * 256 + -(-mb // 256) * 256 + dwb
    assert prefill_size(L, 16, 64, 8193, 64)[1] > prefill_size(L, 16, 64, 8192, 64)[1] - 1
    for bad in (dict(topk=0), dict(s_kv=0), dict(h_kv=2), dict(s_q=0), dict(h_q=0)):
        kw = dict(s_q=16, h_q=64, s_kv=1000, topk=64)
        kw.update(bad)
        rc, _, _ = prefill_size(L, **kw)
        assert rc < 0, bad


def test_noalloc_refuses_shapes_beyond_its_scratch(L):
    """The allocation-free entry point checks the shape's workspace against its
    static scratch on the host and refuses larger ones before any HIP call."""
    f = L.mla_decode_with_kvcache_noalloc
    f.argtypes = None
    P = ctypes.c_void_p
    # 4096 requests x 512 query rows: the split workspace is far beyond 128 MiB
    rc = f(P(0x1000), P(0x2000), ctypes.c_int64(4), P(0x3000), 4, P(0x4000), 4096, 4, 128, 1, 576, 512,
           ctypes.c_float(0.0), P(0x5000), ctypes.c_size_t(1 << 30), 256, None, 0, 0, 0, P(0x7000), P(0x8000), None)
    assert rc == -2
    assert "scratch" in L.mla_last_error().decode()


def test_header_is_plain_c(tmp_path):
    """include/mla_decode.h is a C header: a C99 translation unit that calls
    every declared entry point compiles without warnings (gcc, syntax only)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not installed")
    src = tmp_path / "use_header.c"
    src.write_text("""#include "mla_decode.h"
int main(void) {
  size_t a = 0, b = 0;
  int w = 0;
  int rc = mla_get_metadata_size(1, 1, 16, 1, 0, 8, &a, &b, &w);
  rc |= mla_set_merge_mode(MLA_MERGE_OFF);
  rc |= mla_set_decode_kernel_events(NULL, NULL);
  (void)mla_last_error();
  (void)mla_get_metadata; (void)mla_decode_with_kvcache; (void)mla_decode_with_kvcache_noalloc;
  (void)mla_debug_dequant_fp8; (void)mla_sparse_prefill; (void)mla_sparse_prefill_workspace_size;
  return rc;
}
""")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", inc, "-fsyntax-only", str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
