"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (automatic worker count).  The oracle checks every row of the
tiny dense workload and of the skewed long-context one, and a seeded sample of
rows (covering every request) for the large ones."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from gpu_helpers import check_problem, say

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
