"""The allocation-free entry point (mla_decode_with_kvcache_noalloc) through the
C ABI: its split workspace is the library's static scratch array, so it must give
exactly what mla_decode_with_kvcache gives with a caller workspace, on two calls
in a row where the second has a smaller input (the scratch keeps the first
call's contents), and both within the tolerance of the oracle."""
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import DEV, compare, flat, say, to_device

pytestmark = pytest.mark.gpu


def _both(prob, num_workers):
    import mla_paged_kv_get_amd as mla

    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8, num_workers)
    o_ws, lse_ws = mla.mla_decode_with_kvcache(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta,
                                               d["indices"], prob.is_fp8, prob.softmax_scale)
    o_na = torch.full((prob.B, prob.s_q, prob.h_q, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse_na = torch.full((prob.B, prob.s_q, prob.h_q), float("nan"), dtype=torch.float32, device=DEV)
    mla.mla_decode_with_kvcache_noalloc(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta, o_na,
                                        lse_na, d["indices"], prob.is_fp8, prob.softmax_scale)
    torch.cuda.synchronize()
    return o_ws, lse_ws, o_na, lse_na, meta


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = mi.make_problem("noalloc: sparse fp8, many splits", 4, 1, 128, [3000, 2500, 700, 4000], seed=201,
                          topk=512, is_fp8=True, n_invalid=20)
    small = mi.make_problem("noalloc: dense bf16, smaller", 2, 1, 16, [70, 200], seed=202)
    for prob, W in ((big, 64), (small, 5)):
        say("[gpu] %s (W=%d)" % (prob.name, W))
        o_ws, lse_ws, o_na, lse_na, meta = _both(prob, W)
        assert meta.total_splits() > prob.B * prob.s_q  # the scratch is used: some streams have several splits
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), prob.name
        assert torch.equal(lse_na, lse_ws), prob.name
        o, lse = flat(o_na, lse_na)
        o_ref, lse_ref = oracle.problem_decode(prob)
        compare(o, lse, o_ref, lse_ref, prob.name)


def test_noalloc_in_merge_mode():
    """The allocation-free entry point with the decode kernel merging the splits
    (its partials then live in the static scratch too): the same bits as the
    workspace entry point with the combine kernel."""
    import mla_paged_kv_get_amd as mla

    prob = mi.make_problem("noalloc: dense bf16 merged", 3, 1, 64, [200, 64, 130], seed=203)
    say("[gpu] %s" % prob.name)
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, 0, False, 0)
    o_ws, lse_ws = mla.mla_decode_with_kvcache(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta)
    mla.mla_set_merge_mode(mla.MLA_MERGE_ON)
    try:
        o_na = torch.empty_like(o_ws)
        lse_na = torch.empty_like(lse_ws)
        mla.mla_decode_with_kvcache_noalloc(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta,
                                            o_na, lse_na)
        torch.cuda.synchronize()
    finally:
        mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
    assert meta.total_splits() > prob.B
    assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws)
