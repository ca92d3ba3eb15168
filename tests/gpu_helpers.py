"""Shared helpers of the GPU tests: run a problem through the C ABI and compare
with the float64 oracle at the stated tolerance."""
import sys

import numpy as np
import torch

import oracle

# Floating-point bar: o elementwise |d| <= 8e-3 + 1e-2 |o_ref|, lse |d| <= 1e-3;
# where the oracle says the attended set is empty (lse = -inf) the GPU must give
# lse = -inf and o = 0 exactly.
O_ATOL, O_RTOL, LSE_ATOL = 8e-3, 1e-2, 1e-3

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(prob):
    d = dict(q=prob.q.to(DEV), kvcache=prob.kvcache.to(DEV), block_table=prob.block_table.to(DEV),
             cache_seqlens=prob.cache_seqlens.to(DEV),
             indices=None if prob.indices is None else prob.indices.to(DEV))
    return d


def run_gpu(prob, num_workers=0, dev_inputs=None, meta=None, causal=False):
    import mla_paged_kv_get_amd as mla

    d = dev_inputs or to_device(prob)
    if meta is None:
        meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8, num_workers)
    o, lse = mla.mla_decode_with_kvcache(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta,
                                         d["indices"], prob.is_fp8, prob.softmax_scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, meta


def flat(o, lse):
    o = o.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    return o, lse


def record_margin(what, do, ratio, dl):
    """Keep a case's margins for the terminal summary (conftest.MARGINS)."""
    import conftest

    conftest.MARGINS.append((what, float(do), float(ratio), float(dl)))


def compare(o, lse, o_ref, lse_ref, what=""):
    """Assert the tolerance; returns (max |d o|, max |d lse|) and records them."""
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[empty])), "%s: rows with no attended token must give lse = -inf" % what
    assert np.all(o[empty] == 0.0), "%s: rows with no attended token must give o = 0" % what
    live = ~empty
    do = np.abs(o[live] - o_ref[live])
    bound = O_ATOL + O_RTOL * np.abs(o_ref[live])
    bad = do > bound
    assert not np.any(np.isnan(o[live])), "%s: NaN in o" % what
    assert not bad.any(), "%s: %d/%d o elements out of tolerance, worst |d| %.3g" % (what, bad.sum(), bad.size, do.max())
    dl = np.abs(lse[live] - lse_ref[live])
    assert np.all(dl <= LSE_ATOL), "%s: lse out of tolerance, worst |d| %.3g" % (what, dl.max())
    do_max = float(do.max()) if do.size else 0.0
    dl_max = float(dl.max()) if dl.size else 0.0
    record_margin(what, do_max, float((do / bound).max()) if do.size else 0.0, dl_max)
    return do_max, dl_max


def check_problem(prob, rows=None, num_workers=0, what=None, causal=False):
    """Run on the GPU and compare all rows (rows=None) or a sample with the oracle."""
    what = what or prob.name
    say("[gpu] %s (W=%s%s)" % (what, num_workers or "auto", ", causal" if causal else ""))
    o, lse, _ = run_gpu(prob, num_workers, causal=causal)
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob, rows, causal)
    if rows is not None:
        o, lse = o[rows], lse[rows]
    return compare(o, lse, o_ref, lse_ref, what)
