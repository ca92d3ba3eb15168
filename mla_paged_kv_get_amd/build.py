"""Build the gfx950 HIP library libmla_decode.so in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only; packed fp32 instructions
are disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The kernel
resource report (VGPR/AGPR/SGPR counts, scratch, occupancy) is written to
_build/resource_usage.txt, and the build fails if a kernel uses scratch memory
(register spills), unless MLA_ALLOW_SPILLS=1.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-Rpass-analysis=kernel-resource-usage"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr


def _scratch_report(log: str):
    """(kernel, scratch bytes) for every kernel in a -Rpass-analysis log."""
    out = []
    current = None
    for line in log.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and current:
            out.append((current, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    logs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = []
    for src, obj, rc, log in results:
        log = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
        logs.append("==== %s\n%s" % (os.path.basename(src), log))
        if rc != 0:
            sys.stderr.write(log + "\n")
            raise RuntimeError("hipcc failed on %s" % src)
        objs.append(obj)
    report = "\n".join(logs)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(report)
    spills = [(k, s) for k, s in _scratch_report(report) if s > 0]
    if spills and os.environ.get("MLA_ALLOW_SPILLS") != "1":
        raise RuntimeError("kernels use scratch (register spills): %s" % spills)
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, capture_output=True,
                       text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    # every symbol must resolve (a kernel the host pass failed to emit shows up here)
    import ctypes
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        os.unlink(tmp)
        raise RuntimeError("linked library does not load: %s" % e)
    os.replace(tmp, LIB)
    if verbose:
        print(report)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
