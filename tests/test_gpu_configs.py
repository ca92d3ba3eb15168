"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (automatic worker count).  The oracle checks every row of the
tiny dense workload and of the skewed long-context one, and a seeded sample of
rows (covering every request) for the large ones."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import check_problem, compare, flat, run_gpu, say

pytestmark = pytest.mark.gpu

SAMPLE = {1: None, 2: 256, 3: 160, 4: 256, 5: None}


def sample_rows(prob, n, seed):
    rows_per_req = prob.s_q * prob.h_q
    total = prob.B * rows_per_req
    rng = np.random.default_rng(seed)
    # one row from every request, then random rows
    first = np.arange(prob.B) * rows_per_req + rng.integers(0, rows_per_req, prob.B)
    extra = rng.choice(total, size=max(0, n - prob.B), replace=False)
    return np.unique(np.concatenate([first, extra, [0, total - 1]]))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_parity(cfg):
    say("[gpu] building workload %d" % cfg)
    prob = mi.config(cfg)
    rows = None if SAMPLE[cfg] is None else sample_rows(prob, SAMPLE[cfg], cfg)
    do, dl = check_problem(prob, rows=rows, what="workload %d: %s" % (cfg, prob.name))
    say("[gpu] workload %d max |d o| %.3g max |d lse| %.3g" % (cfg, do, dl))
    if cfg == 3:
        # the speculative (s_q = 2) dense workload with the causal mask
        do, dl = check_problem(prob, rows=rows, what="workload 3 causal", causal=True)
        say("[gpu] workload 3 causal max |d o| %.3g max |d lse| %.3g" % (do, dl))
    torch.cuda.empty_cache()


def attended_counts(prob, causal=False):
    """Exact number of attended tokens of every query row ((b * s_q + s) * h_q + h)."""
    sl = prob.cache_seqlens.numpy().astype(np.int64)
    if prob.indices is not None:
        per_bs = (prob.indices.numpy() != -1).sum(axis=2).reshape(-1)
    else:
        s = np.arange(prob.s_q)
        if causal:
            per = np.clip(sl[:, None] - prob.s_q + s[None, :] + 1, 0, sl[:, None])
        else:
            per = np.broadcast_to(sl[:, None], (prob.B, prob.s_q))
        per_bs = per.reshape(-1)
    return np.repeat(per_bs, prob.h_q).astype(np.float64)


COVERAGE = [(1, False), (2, False), (3, False), (3, True), (4, False), (5, False)]


@pytest.mark.parametrize("cfg,causal", COVERAGE, ids=["c%d%s" % (c, " causal" if k else "") for c, k in COVERAGE])
def test_full_size_coverage(cfg, causal):
    """With q = 0 every score is 0, so each row's weights are uniform: exp(lse) is
    exactly the number |T| of tokens the row attends and o is the mean of V over
    T.  At full size, in the launch configuration the benchmark times, every row
    must give |exp(lse) - |T|| < 0.5 (a token dropped or counted twice moves
    exp(lse) by 1), and o must match the oracle's mean within the tolerance."""
    c = dict(mi.CONFIGS[cfg])
    name = c.pop("name")
    say("[gpu] coverage (q = 0) workload %d%s" % (cfg, " causal" if causal else ""))
    prob = mi.make_problem("coverage " + name, seed=cfg, q_zero=True, **c)
    counts = attended_counts(prob, causal)
    o, lse, _ = run_gpu(prob, causal=causal)
    o, lse = flat(o, lse)
    # q = 0 gives every head of a (request, query token) the same result: the
    # oracle evaluates one row per (b, s)
    rep = np.arange(prob.B * prob.s_q) * prob.h_q
    o_bs, lse_bs = oracle.problem_decode(prob, rep, causal)
    live_bs = counts[rep] > 0
    assert np.allclose(lse_bs[live_bs], np.log(counts[rep][live_bs]), rtol=0, atol=1e-12)
    o_ref = np.repeat(o_bs, prob.h_q, axis=0)
    lse_ref = np.repeat(lse_bs, prob.h_q)
    what = "coverage c%d%s" % (cfg, " causal" if causal else "")
    do, dl = compare(o, lse, o_ref, lse_ref, what)
    live = counts > 0
    err = np.abs(np.exp(lse[live]) - counts[live])
    say("[gpu] %s: %d rows, |T| %d..%d, max |exp(lse) - |T|| %.3g, max |d o| %.3g" % (
        what, live.sum(), counts[live].min(), counts[live].max(), err.max(), do))
    assert err.max() < 0.5, "%s: a row attended a different number of tokens (max |exp(lse) - |T|| %.3g)" % (
        what, err.max())
    del prob
    torch.cuda.empty_cache()
