"""GPU: decode calls that merge their splits in the decode kernel (the last split
of each row tile folds the stream's split results by their lse and writes o and
lse; no combine launch).  The merged result must be bit-identical to the
separate combine kernel's, match the oracle, survive repeated calls on one
metadata buffer (the arrival counters reset themselves) and fill empty dense
streams with o = 0, lse = -inf."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import DEV, compare, flat, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _auto_mode_after():
    yield
    import mla_paged_kv_get_amd as mla

    mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)


# (problem, worker count): every stream has at most 4 splits, some have 2 or more
CASES = [
    (dict(name="dense bf16 h64 with an empty request", B=4, s_q=1, h_q=64, seqlens=[200, 64, 130, 0], seed=141), 0),
    (dict(name="dense fp8 h128 (2 row tiles)", B=2, s_q=1, h_q=128, seqlens=[700, 300], seed=142, is_fp8=True), 0),
    (dict(name="dense bf16 causal s_q=2 h64 (2 row tiles)", B=2, s_q=2, h_q=64, seqlens=[513, 77], seed=143,
          causal=True), 0),
    (dict(name="dense bf16 h16 long, 3 workers", B=2, s_q=1, h_q=16, seqlens=[3000, 1000], seed=144), 3),
    (dict(name="sparse bf16 s_q=2 h64", B=3, s_q=2, h_q=64, seqlens=[900, 600, 2000], topk=512, n_invalid=20,
          seed=145), 16),
    (dict(name="sparse fp8 h128", B=2, s_q=1, h_q=128, seqlens=[5000, 1500], topk=1024, n_invalid=30, is_fp8=True,
          seed=146), 4),
    (dict(name="sparse fp8 h40 (partial row tile) s_q=3", B=2, s_q=3, h_q=40, seqlens=[900, 400], topk=320,
          n_invalid=9, is_fp8=True, seed=147), 9),
    (dict(name="sparse bf16 padded lists (empty splits)", B=2, s_q=1, h_q=64, seqlens=[3000, 200], topk=1024,
          recipe="clip", seed=148), 4),
]


def _split_counts(prob, meta):
    m = meta.tensor.cpu().numpy()
    W = int(m[2])
    _, off = oracle.schedule(prob.cache_seqlens.numpy(), prob.s_q, prob.topk, W, int(m[7]))
    return np.diff(off)


def _arrive_slice(prob, meta):
    m = meta.tensor
    W, n = int(m[2].item()), int(m[1].item())
    R = prob.h_q if prob.topk else prob.s_q * prob.h_q
    start = 16 + 8 * W + 2 * (n + 1)
    return m[start:start + n * ((R + 63) // 64)]


def _call(mla, prob, d, meta, causal, ws=None, o=None, lse=None):
    o_, l_ = mla.mla_decode_with_kvcache(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta,
                                         d["indices"], prob.is_fp8, prob.softmax_scale, ws, o, lse, causal=causal)
    torch.cuda.synchronize()
    return o_.clone(), l_.clone()


@pytest.mark.parametrize("case,W", CASES, ids=[c[0]["name"] for c in CASES])
def test_merged_equals_combine_kernel_and_oracle(case, W):
    import mla_paged_kv_get_amd as mla

    c = dict(case)
    causal = c.pop("causal", False)
    prob = mi.make_problem(c.pop("name"), **c)
    say("[gpu] merge: %s (W=%s)" % (prob.name, W or "auto"))
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8, W)
    splits = _split_counts(prob, meta)
    assert splits.max() <= 4 and splits.max() >= 2, splits
    mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
    o0, l0 = _call(mla, prob, d, meta, causal)
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    ws = torch.full((meta.workspace_bytes,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN bytes
    o1, l1 = _call(mla, prob, d, meta, causal, ws=ws)
    assert torch.equal(o1, o0) and torch.equal(l1, l0), "merged result differs from the combine kernel's"
    # the same metadata again: the counters were reset by the merging splits
    for _ in range(2):
        o2, l2 = _call(mla, prob, d, meta, causal)
        assert torch.equal(o2, o0) and torch.equal(l2, l0)
    assert int(_arrive_slice(prob, meta).abs().sum().item()) == 0
    o, lse = flat(o1, l1)
    o_ref, lse_ref = oracle.problem_decode(prob, None, causal)
    compare(o, lse, o_ref, lse_ref, "merged " + prob.name)
    # new queries on the same metadata and workspace: a merge that read a
    # split's partial left from the previous call would mix the two
    d2 = dict(d)
    d2["q"] = torch.flip(d["q"], dims=[2]).contiguous()
    mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
    o3, l3 = _call(mla, prob, d2, meta, causal, ws=ws)
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    _call(mla, prob, d, meta, causal, ws=ws)
    o4, l4 = _call(mla, prob, d2, meta, causal, ws=ws)
    assert torch.equal(o4, o3) and torch.equal(l4, l3), "merged call used partials of an earlier call"
    assert not torch.equal(o3, o0)


def test_merge_is_taken_and_counted():
    """With every arrival counter set far from its stream's split count, no split
    is last, so nothing merges: the rows of split streams keep what o held
    before (NaN here), which shows that the call took the merging path and
    launched no combine; single-split streams are written as usual."""
    import mla_paged_kv_get_amd as mla

    prob = mi.make_problem("merge counters", 3, 1, 64, [200, 64, 130], seed=149)
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, 0, False, 0)
    splits = _split_counts(prob, meta)
    assert list(splits > 1) == [True, False, True], splits
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    _arrive_slice(prob, meta).fill_(1000)
    o = torch.full((3, 1, 64, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((3, 1, 64), float("nan"), dtype=torch.float32, device=DEV)
    _call(mla, prob, d, meta, False, o=o, lse=lse)
    assert torch.isnan(o[0]).all() and torch.isnan(o[2]).all() and torch.isnan(lse[0]).all()
    o_ref, lse_ref = oracle.problem_decode(prob, None, False)
    got, gl = flat(o[1:2], lse[1:2])
    compare(got, gl, o_ref.reshape(3, 64, 512)[1], lse_ref.reshape(3, 64)[1], "single-split stream")
    assert (_arrive_slice(prob, meta) == 1000 + torch.tensor([splits[0], 0, splits[2]], device=DEV,
                                                             dtype=torch.int32)).all()


def test_default_mode_launches_the_combine():
    """By default a decode call does not merge in the decode kernel even where it
    could (the tiny workload): poisoned arrival counters change nothing, and
    the result equals the merged one."""
    import mla_paged_kv_get_amd as mla

    prob = mi.config(1)
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, 0, False, 0)
    assert _split_counts(prob, meta).max() >= 2
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    o1, l1 = _call(mla, prob, d, meta, False)
    mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
    _arrive_slice(prob, meta).fill_(1000)
    o0, l0 = _call(mla, prob, d, meta, False)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    o, lse = flat(o0, l0)
    o_ref, lse_ref = oracle.problem_decode(prob)
    compare(o, lse, o_ref, lse_ref, "tiny workload, combine kernel")


@pytest.mark.parametrize("kw,W", [
    (dict(B=2, s_q=1, h_q=64, seqlens=[700, 200]), 0),                      # dense: max_blocks 11, splits of 2 tiles
    (dict(B=2, s_q=1, h_q=64, seqlens=[3000, 1500], topk=1024), 64),        # sparse: 16 tiles per stream, q = 2
], ids=["dense long rows", "sparse many splits"])
def test_merge_mode_falls_back_where_unproven(kw, W):
    """Where the host cannot prove at most 4 splits per stream, a call in merge
    mode runs the combine kernel: poisoned arrival counters change nothing."""
    import mla_paged_kv_get_amd as mla

    prob = mi.make_problem("merge fallback", seed=150, **kw)
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8, W)
    mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
    o0, l0 = _call(mla, prob, d, meta, False)
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    _arrive_slice(prob, meta).fill_(1000)
    o1, l1 = _call(mla, prob, d, meta, False)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    assert (_arrive_slice(prob, meta) == 1000).all()
