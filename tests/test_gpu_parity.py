"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bit-exact: the FP8 -> bf16 decode, the metadata (against the oracle's plain
schedule rule) and the page indirection (permuting pages gives identical
bits).  Floating point: o within 8e-3 + 1e-2 |o_ref| elementwise, lse within
1e-3, -inf / 0 exactly for empty attended sets.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import DEV, check_problem, compare, flat, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import mla_paged_kv_get_amd as mla

    mla.lib()
    assert torch.cuda.is_available(), "GPU tests need the MI355X"


# --------------------------------------------------------------------------------------
# bit-exact pieces


def test_fp8_decode_bit_exact():
    import mla_paged_kv_get_amd as mla

    say("[gpu] fp8 decode: 256 codes x 12 scales")
    scales = np.array([1.0, 0.0023, 3.7e-5, 448.0 / 7.0, 1.5e-38, 2.0 ** -120, 0.1, 7.0, 1e-3, 123.456, 2.0 ** -126,
                       0.0], dtype=np.float32)
    n = 256 * 3
    tok = np.zeros((n, 656), dtype=np.uint8)
    rng = np.random.default_rng(0)
    for t in range(n):
        tok[t, :512] = (np.arange(512) + t) % 256
        tok[t, 512:528] = scales[(np.arange(4) + t) % len(scales)].view(np.uint8)
        tok[t, 528:] = rng.integers(0, 256, 128, dtype=np.uint8)
    got = mla.mla_debug_dequant_fp8(torch.from_numpy(tok).to(DEV)).cpu().view(torch.int16).numpy().view(np.uint16)
    torch.cuda.synchronize()
    for t in range(n):
        sc = tok[t, 512:528].view(np.float32)
        want = oracle.fp8_dequant_bf16(tok[t, :512], np.repeat(sc, 128))
        nan = (tok[t, :512] & 0x7F) == 0x7F
        g = got[t, :512]
        assert np.array_equal(g[~nan], want[~nan]), "token %d" % t
        assert np.all(((g[nan] & 0x7F80) == 0x7F80) & ((g[nan] & 0x7F) != 0))
        assert np.array_equal(got[t, 512:], tok[t, 528:].view(np.uint16))


@pytest.mark.parametrize("seed", range(4))
def test_metadata_matches_schedule_rule(seed):
    import mla_paged_kv_get_amd as mla

    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 50))
    s_q = int(rng.integers(1, 3))
    topk = int(rng.choice([0, 0, 64, 2048]))
    seqlens = rng.integers(0, 9000, size=B).astype(np.int32)
    seqlens[rng.random(B) < 0.2] = 0
    W = int(rng.choice([1, 7, 64, 256, 1000]))
    say("[gpu] metadata B=%d s_q=%d topk=%d W=%d" % (B, s_q, topk, W))
    meta = mla.mla_get_metadata(torch.from_numpy(seqlens).to(DEV), s_q, 64, 1, topk, False, W)
    m = meta.tensor.cpu().numpy()
    torch.cuda.synchronize()
    n_streams = B * s_q if topk else B
    assert m[1] == n_streams and m[2] == W
    sched_ref, off_ref = oracle.schedule(seqlens, s_q, topk, W, int(m[7]))
    assert np.array_equal(m[16:16 + 8 * W].reshape(W, 8), sched_ref)
    assert np.array_equal(m[16 + 8 * W:16 + 8 * W + n_streams + 1], off_ref)
    assert m[5] == off_ref[-1]


@pytest.mark.parametrize("B,s_q,topk,W", [(3000, 1, 0, 256), (700, 2, 2048, 512), (12000, 1, 64, 1024),
                                        (257, 1, 0, 3)])
def test_metadata_many_streams(B, s_q, topk, W):
    """Streams spread over several per-thread chunks, and (above 8192 streams) the
    prefix arrays built in global memory instead of LDS."""
    import mla_paged_kv_get_amd as mla

    rng = np.random.default_rng(B + W)
    seqlens = rng.integers(0, 5000, size=B).astype(np.int32)
    seqlens[rng.random(B) < 0.1] = 0
    say("[gpu] metadata many streams B=%d s_q=%d topk=%d W=%d" % (B, s_q, topk, W))
    meta = mla.mla_get_metadata(torch.from_numpy(seqlens).to(DEV), s_q, 64, 1, topk, False, W)
    m = meta.tensor.cpu().numpy()
    n_streams = B * s_q if topk else B
    sched_ref, off_ref = oracle.schedule(seqlens, s_q, topk, W, int(m[7]))
    assert np.array_equal(m[16:16 + 8 * W].reshape(W, 8), sched_ref)
    assert np.array_equal(m[16 + 8 * W:16 + 8 * W + n_streams + 1], off_ref)


# --------------------------------------------------------------------------------------
# small parity cases: several tiles, ragged tails, every variant


SMALL = [
    dict(name="dense bf16 h16 ragged", B=3, s_q=1, h_q=16, seqlens=[1, 200, 64], seed=1),
    dict(name="dense bf16 h128", B=2, s_q=1, h_q=128, seqlens=[300, 1000], seed=2),
    dict(name="dense bf16 s_q=2 h64 (128 rows)", B=2, s_q=2, h_q=64, seqlens=[513, 77], seed=3),
    dict(name="dense bf16 s_q=2 h128 (256 rows)", B=2, s_q=2, h_q=128, seqlens=[700, 129], seed=4),
    dict(name="dense fp8 h64", B=2, s_q=1, h_q=64, seqlens=[450, 65], seed=5, is_fp8=True),
    dict(name="sparse bf16 h128", B=2, s_q=1, h_q=128, seqlens=[3000, 500], seed=6, topk=256, n_invalid=13),
    dict(name="sparse fp8 h128", B=3, s_q=1, h_q=128, seqlens=[5000, 2500, 700], seed=7, topk=512, is_fp8=True,
         n_invalid=25),
    dict(name="sparse fp8 s_q=2 h64 clip", B=2, s_q=2, h_q=64, seqlens=[2000, 100], seed=8, topk=300, is_fp8=True,
         recipe="clip"),
    dict(name="sparse fp8 h16 topk 40", B=2, s_q=1, h_q=16, seqlens=[90, 60], seed=9, topk=40, is_fp8=True,
         recipe="clip"),
    dict(name="dense bf16 h96 (partial row tile)", B=2, s_q=1, h_q=96, seqlens=[333, 64], seed=10),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["name"] for c in SMALL])
def test_small_parity(case):
    c = dict(case)
    prob = mi.make_problem(c.pop("name"), **c)
    check_problem(prob)


@pytest.mark.parametrize("W", [1, 7, 256, 1000])
def test_forced_worker_counts(W):
    prob = mi.make_problem("dense bf16 splits", 3, 1, 64, [2000, 64, 700], seed=21)
    check_problem(prob, num_workers=W, what="dense W=%d" % W)
    sp = mi.make_problem("sparse fp8 splits", 2, 2, 64, [4000, 900], seed=22, topk=600, is_fp8=True, recipe="clip")
    check_problem(sp, num_workers=W, what="sparse fp8 W=%d" % W)


@pytest.mark.parametrize("is_fp8,topk,W", [(False, 0, 256), (True, 0, 96), (False, 4096, 256), (True, 4096, 64)],
                         ids=["dense bf16 W=256", "dense fp8 W=96", "sparse bf16 W=256", "sparse fp8 W=64"])
def test_many_splits_per_stream(is_fp8, topk, W):
    """Long streams cut into 32-64 splits: the combine kernel's path for more
    splits than it loads at once (lse values first, then the split outputs
    eight at a time), next to a short stream (dense) or a second long one
    (sparse); the combine variant that loads 16 splits at once."""
    prob = mi.make_problem("many splits", 2, 1, 32, [8192, 100], seed=130 + W, topk=topk, is_fp8=is_fp8,
                           n_invalid=40 if topk else 0, recipe="clip")
    import mla_paged_kv_get_amd as mla

    m = mla.mla_get_metadata(prob.cache_seqlens.to(DEV), 1, 32, 1, topk, is_fp8, W)
    mm = m.tensor.cpu().numpy()
    n = np.diff(mm[16 + 8 * W:16 + 8 * W + 3])
    say("[gpu] many splits W=%d: splits per stream %s" % (W, list(n)))
    assert n.max() > 16
    check_problem(prob, num_workers=W, what="many splits %s topk=%d W=%d" % ("fp8" if is_fp8 else "bf16", topk, W))


def test_combine_over_many_streams():
    """2048 sparse streams of 64 rows (more than 8 passes of the chip at one
    workgroup per 4 rows): the combine kernel's capped grid, each workgroup
    looping over several row groups; 250 workers put split points inside
    streams, so some streams are merged while most are finished by the decode
    kernel.  Checked on a seeded sample of rows that includes every row of the
    merged streams."""
    import mla_paged_kv_get_amd as mla

    prob = mi.make_problem("many streams", 1024, 2, 64, [200] * 1024, seed=151, topk=128, n_invalid=3,
                           recipe="clip")
    m = mla.mla_get_metadata(prob.cache_seqlens.to(DEV), 2, 64, 1, 128, False, 250)
    mm = m.tensor.cpu().numpy()
    n = np.diff(mm[16 + 8 * 250:16 + 8 * 250 + 2048 + 1])
    merged = np.nonzero(n > 1)[0]
    say("[gpu] many streams: %d of 2048 streams merged" % merged.size)
    assert 0 < merged.size < 2048
    rng = np.random.default_rng(151)
    rows = set((merged[:, None] * 64 + np.arange(64)[None, :]).reshape(-1).tolist())
    rows |= set(rng.choice(2048 * 64, size=512, replace=False).tolist())
    check_problem(prob, rows=np.array(sorted(rows)), num_workers=250, what="2048 streams, capped combine grid")


def test_many_splits_among_short_streams():
    """One 8192-token stream among fifteen one-tile streams, 128 workers: the
    combine variant that loads 8 splits at once takes its looping path for the
    long stream's 64 splits."""
    prob = mi.make_problem("many splits among short", 16, 1, 32, [8192] + [64] * 15, seed=141)
    check_problem(prob, num_workers=128, what="64 splits among one-split streams")


@pytest.mark.parametrize("is_fp8,topk", [(False, 0), (True, 0), (False, 320), (True, 320)],
                         ids=["dense bf16", "dense fp8", "sparse bf16", "sparse fp8"])
@pytest.mark.parametrize("W", [5, 19, 61, 150])
def test_split_lengths_every_variant(is_fp8, topk, W):
    """Worker counts that cut the streams into splits of one to several 32-token
    sub-tiles (odd and even counts), for each kernel variant: the pipeline's
    prologue, its main loop and its last rounds all see short and long splits."""
    prob = mi.make_problem("splits", 3, 1, 64, [1500, 333, 770], seed=40 + W, topk=topk, is_fp8=is_fp8,
                           n_invalid=7 if topk else 0, recipe="clip")
    check_problem(prob, num_workers=W, what="%s topk=%d W=%d" % ("fp8" if is_fp8 else "bf16", topk, W))


@pytest.mark.parametrize("is_fp8,topk", [(False, 0), (True, 0), (False, 320), (True, 320)],
                         ids=["dense bf16", "dense fp8", "sparse bf16", "sparse fp8"])
@pytest.mark.parametrize("s_q,W", [(1, 3), (3, 7)])
def test_partial_row_tiles_every_variant(is_fp8, topk, s_q, W):
    """40 query heads: each stream's last (or only) 64-row tile is partial, so Q
    rows past the stream load as zeros and only the existing rows are written
    back; few workers, so a workgroup runs several pieces (streams) in turn."""
    prob = mi.make_problem("partial rows", 3, s_q, 40, [900, 95, 400], seed=60 + W, topk=topk, is_fp8=is_fp8,
                           n_invalid=5 if topk else 0, recipe="clip")
    check_problem(prob, num_workers=W, what="%s topk=%d s_q=%d W=%d" % ("fp8" if is_fp8 else "bf16", topk, s_q, W))


# --------------------------------------------------------------------------------------
# edge cases


def test_empty_streams_and_all_masked():
    prob = mi.make_problem("dense with empty request", 3, 1, 16, [0, 100, 0], seed=31, max_blocks=2)
    check_problem(prob, num_workers=5)
    sp = mi.make_problem("sparse all -1", 2, 1, 64, [300, 300], seed=32, topk=128)
    sp.indices[1] = -1
    sp.indices[0, 0, 5:] = -1
    check_problem(sp, num_workers=3)


EMPTY_SPLITS = [
    # index lists padded with -1 past short requests: whole splits attend nothing
    # (16 or 32 splits per stream: the combine's batched and per-row paths)
    dict(name="sparse bf16 padded lists", B=2, s_q=1, h_q=64, seqlens=[5000, 700], topk=4096, recipe="clip",
         seed=131),
    dict(name="sparse fp8 padded lists", B=2, s_q=2, h_q=64, seqlens=[3000, 500], topk=2048, recipe="clip",
         is_fp8=True, seed=132),
    dict(name="sparse fp8 h128 padded lists", B=3, s_q=1, h_q=128, seqlens=[2100, 90, 1000], topk=2048,
         recipe="clip", is_fp8=True, seed=133),
    # 65 causal query tokens x 2 heads (3 row tiles, so splits of 4 tiles): query
    # token i sees positions <= seqlen - 65 + i, so the first ~20 see nothing of
    # the split that starts at position 256 and the others do
    dict(name="dense bf16 causal 130 rows", B=2, s_q=65, h_q=2, seqlens=[300, 290], seed=134, causal=True),
    dict(name="dense fp8 causal 130 rows", B=2, s_q=65, h_q=2, seqlens=[300, 270], seed=135, is_fp8=True,
         causal=True),
]


@pytest.mark.parametrize("case", EMPTY_SPLITS, ids=[c["name"] for c in EMPTY_SPLITS])
@pytest.mark.parametrize("W", [16, 64, 256])
def test_empty_split_rows_with_nan_workspace(case, W):
    """A split row that attends no token writes only its lse (-inf); its partial
    output stays as the workspace held it (here NaN bytes), and the combine must
    give it weight 0 without touching the result."""
    import mla_paged_kv_get_amd as mla

    c = dict(case)
    causal = c.pop("causal", False)
    prob = mi.make_problem(c.pop("name"), **c)
    say("[gpu] %s (W=%d, NaN workspace)" % (prob.name, W))
    d = to_device(prob)
    meta = mla.mla_get_metadata(d["cache_seqlens"], prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8, W)
    ws = torch.full((meta.workspace_bytes,), 0xFF, dtype=torch.uint8, device=DEV)
    o, lse = mla.mla_decode_with_kvcache(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, meta,
                                         d["indices"], prob.is_fp8, prob.softmax_scale, workspace=ws, causal=causal)
    torch.cuda.synchronize()
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob, None, causal)
    compare(o, lse, o_ref, lse_ref, "%s W=%d" % (prob.name, W))


@pytest.mark.parametrize("is_fp8", [False, True])
def test_single_token(is_fp8):
    prob = mi.make_problem("single token", 1, 1, 64, [300], seed=41, topk=64, is_fp8=is_fp8)
    prob.indices[0, 0] = -1
    prob.indices[0, 0, 17] = 233
    o, lse, _ = run_gpu(prob)
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob)
    assert np.array_equal(o, o_ref)  # p = 1: o is the token's V, bf16 exactly
    compare(o, lse, o_ref, lse_ref, "single token")


@pytest.mark.parametrize("is_fp8,topk", [(False, 0), (True, 0), (False, 200), (True, 200)])
def test_unattended_nan_never_leaks(is_fp8, topk):
    kw = dict(B=2, s_q=1, h_q=64, seqlens=[330, 100], seed=51, is_fp8=is_fp8, topk=topk, n_spare=3, max_blocks=8)
    if topk:
        kw.update(recipe="clip", n_invalid=10)
    prob = mi.make_problem("nan-poisoned", nan_fill=True, **kw)
    check_problem(prob, num_workers=4)


def test_page_permutation_bit_identical():
    prob = mi.make_problem("perm", 2, 1, 128, [900, 300], seed=61, n_spare=5)
    o1, l1, _ = run_gpu(prob, 4)
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(prob.num_blocks, generator=g)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    prob.kvcache = prob.kvcache[perm].contiguous()
    prob.block_table = inv[prob.block_table.to(torch.int64)].to(torch.int32)
    o2, l2, _ = run_gpu(prob, 4)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_dense_equals_sparse_full_list():
    dense = mi.make_problem("d", 2, 1, 64, [150, 64], seed=71)
    sparse = mi.make_problem("d", 2, 1, 64, [150, 64], seed=71)
    idx = torch.full((2, 1, 192), -1, dtype=torch.int32)
    for b, L in enumerate([150, 64]):
        idx[b, :, :L] = torch.arange(L, dtype=torch.int32)
    sparse.indices = idx
    od, ld, _ = run_gpu(dense, 2)
    os_, ls, _ = run_gpu(sparse, 2)
    o, lse = flat(od, ld)
    o2, lse2 = flat(os_, ls)
    o_ref, lse_ref = oracle.problem_decode(dense)
    compare(o, lse, o_ref, lse_ref, "dense")
    compare(o2, lse2, o_ref, lse_ref, "sparse as dense")


def test_deterministic():
    prob = mi.make_problem("det", 4, 1, 128, [1500, 20, 800, 64], seed=81, is_fp8=True, topk=256, n_invalid=9,
                           recipe="clip")
    d = to_device(prob)
    o1, l1, m = run_gpu(prob, dev_inputs=d)
    o2, l2, _ = run_gpu(prob, dev_inputs=d, meta=m)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_metadata_reused_across_calls():
    """One metadata buffer serves many decode calls (one per layer): the decode
    and combine kernels only read it, so repeated calls give the same result."""
    prob = mi.make_problem("reuse", 5, 1, 128, [0, 2000, 700, 64, 1500], seed=85, max_blocks=32)
    d = to_device(prob)
    o_ref, lse_ref = oracle.problem_decode(prob)
    m = None
    for call in range(3):
        o, l, m = run_gpu(prob, 1000, dev_inputs=d, meta=m)
        o, l = flat(o, l)
        compare(o, l, o_ref, lse_ref, "call %d with shared metadata" % call)


@pytest.mark.parametrize("is_fp8,topk,scale", [(False, 0, 4.0), (True, 0, 4.0), (False, 256, 4.0), (True, 256, 4.0)])
def test_large_score_spread(is_fp8, topk, scale):
    """Scores spread over hundreds of natural-log units: later tokens overflow the
    first sub-tile's reference, so the split must be recomputed with the true
    maximum, which in turn must be taken over every token of each row."""
    kw = dict(seed=95, is_fp8=is_fp8, softmax_scale=scale)
    if topk:
        kw.update(topk=topk, n_invalid=7)
    prob = mi.make_problem("large spread", 2, 1, 128, [2000, 700], **kw)
    check_problem(prob, num_workers=3)


def test_lse_merge_through_the_abi():
    """Two calls over the two halves of each index list, merged with the oracle's
    lse rule, equal one call over the whole list."""
    prob = mi.make_problem("halves", 2, 1, 64, [3000, 3000], seed=91, topk=512, is_fp8=True, n_invalid=30)
    o, lse, _ = run_gpu(prob)
    o, lse = flat(o, lse)
    parts = []
    for half in range(2):
        p2 = mi.make_problem("halves", 2, 1, 64, [3000, 3000], seed=91, topk=512, is_fp8=True, n_invalid=30)
        p2.indices = p2.indices.clone()
        p2.indices[:, :, half * 256:(half + 1) * 256] = -1
        oh, lh, _ = run_gpu(p2)
        parts.append(flat(oh, lh))
    merged_o = np.zeros_like(o)
    merged_l = np.zeros_like(lse)
    for r in range(o.shape[0]):
        mo, ml = oracle.lse_combine(np.stack([parts[0][0][r], parts[1][0][r]]), np.array([parts[0][1][r], parts[1][1][r]]))
        merged_o[r], merged_l[r] = mo, ml
    o_ref, lse_ref = oracle.problem_decode(prob)
    compare(merged_o, merged_l, o_ref, lse_ref, "merged halves")
    compare(o, lse, o_ref, lse_ref, "whole")


# --------------------------------------------------------------------------------------
# causal masking for speculative query tokens (dense): query token s of s_q sees cache
# positions <= seqlen - s_q + s


CAUSAL = [
    dict(name="causal bf16 s_q=2 h64, windows of 0 and 1 token", B=4, s_q=2, h_q=64, seqlens=[513, 77, 1, 2], seed=91),
    dict(name="causal bf16 s_q=4 h32", B=3, s_q=4, h_q=32, seqlens=[200, 3, 64], seed=92),
    dict(name="causal fp8 s_q=3 h64", B=2, s_q=3, h_q=64, seqlens=[450, 65], seed=93, is_fp8=True),
    dict(name="causal bf16 s_q=2 h128 (256 rows)", B=2, s_q=2, h_q=128, seqlens=[700, 129], seed=94),
]


@pytest.mark.parametrize("case", CAUSAL, ids=[c["name"] for c in CAUSAL])
@pytest.mark.parametrize("W", [0, 7])
def test_causal_parity(case, W):
    c = dict(case)
    prob = mi.make_problem(c.pop("name"), **c)
    check_problem(prob, num_workers=W, causal=True)


def test_causal_one_query_token_is_bit_identical_to_noncausal():
    prob = mi.make_problem("causal s_q=1", 3, 1, 64, [300, 64, 1000], seed=95)
    d = to_device(prob)
    o1, l1, _ = run_gpu(prob, 0, dev_inputs=d, causal=True)
    o0, l0, _ = run_gpu(prob, 0, dev_inputs=d)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_causal_rejected_for_sparse():
    import mla_paged_kv_get_amd as mla

    prob = mi.make_problem("causal sparse", 1, 2, 16, [300], seed=96, topk=64)
    with pytest.raises(mla.MlaError, match="causal"):
        run_gpu(prob, 0, causal=True)


# --------------------------------------------------------------------------------------
# sparse prefill: many query tokens over one contiguous KV sequence, through the
# same sparse path (the oracle sees it as one request with an identity page table)

PREFILL = [
    dict(name="prefill s_q=48 h64", s_q=48, h_q=64, s_kv=700, topk=128, n_invalid=5, seed=101),
    dict(name="prefill h128 topk past s_kv (clip)", s_q=20, h_q=128, s_kv=100, topk=256, recipe="clip", seed=102),
    dict(name="prefill h40 partial rows", s_q=33, h_q=40, s_kv=3000, topk=512, n_invalid=9, seed=103),
]


@pytest.mark.parametrize("case", PREFILL, ids=[c["name"] for c in PREFILL])
@pytest.mark.parametrize("W", [0, 7])
def test_sparse_prefill(case, W):
    import mla_paged_kv_get_amd as mla

    c = dict(case)
    prob = mi.make_prefill_problem(c.pop("name"), **c)
    say("[gpu] %s (W=%s)" % (prob.name, W or "auto"))
    dev = torch.device("cuda:0")
    s_kv = int(prob.cache_seqlens[0])
    q = prob.q[0].to(dev)
    kv = prob.kvcache.reshape(-1, 576)[:s_kv].contiguous().to(dev)
    idx = prob.indices[0].to(dev)
    o, lse = mla.mla_sparse_prefill(q, kv, idx, softmax_scale=prob.softmax_scale, num_workers=W)
    torch.cuda.synchronize()
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob)
    compare(o, lse, o_ref, lse_ref, prob.name)


def test_sparse_bf16_pool_past_4gib():
    """Sparse BF16 gathers from pools under 4 GiB go through one buffer resource
    over the pool; larger pools take per-lane addresses.  The same problem's pages
    placed at the top of a 4.3 GB pool (so every gathered token lies past 4 GiB)
    must give the oracle's result too."""
    prob = mi.make_problem("sparse bf16 in a 4.3 GB pool", 2, 1, 64, [900, 300], seed=111, topk=192, n_invalid=11)
    d = to_device(prob)
    n = prob.num_blocks
    big_pages = (int(4.3e9) // (64 * 576 * 2)) + n
    big = torch.empty((big_pages, 64, 576), dtype=torch.bfloat16, device=DEV)
    big[big_pages - n:] = d["kvcache"]
    d["kvcache"] = big
    d["block_table"] = d["block_table"] + (big_pages - n)
    say("[gpu] %s (%d pages, %.2f GB)" % (prob.name, big_pages, big.numel() * 2 / 1e9))
    o, lse, _ = run_gpu(prob, num_workers=5, dev_inputs=d)
    del big, d
    torch.cuda.empty_cache()
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob)
    compare(o, lse, o_ref, lse_ref, prob.name)


@pytest.mark.parametrize("topk", [0, 192])
def test_fp8_pool_past_4gib(topk):
    """FP8 token loads from pools whose byte offsets fit 32 bits go through one
    buffer resource over the pool (unattended tokens read past its end); larger
    pools take per-token addresses and a zero token.  The same problem's pages at
    the top of a 4.3 GB FP8 pool must give the oracle's result too (dense and
    sparse)."""
    kind = "sparse" if topk else "dense"
    prob = mi.make_problem("%s fp8 in a 4.3 GB pool" % kind, 2, 1, 64, [900, 300], seed=112 + topk, topk=topk,
                           is_fp8=True, n_invalid=11 if topk else 0)
    d = to_device(prob)
    n = prob.num_blocks
    page_bytes = d["kvcache"][0].numel() * d["kvcache"].element_size()
    big_pages = (int(4.3e9) // page_bytes) + n
    big = torch.empty((big_pages,) + tuple(d["kvcache"].shape[1:]), dtype=d["kvcache"].dtype, device=DEV)
    big[big_pages - n:] = d["kvcache"]
    d["kvcache"] = big
    d["block_table"] = d["block_table"] + (big_pages - n)
    say("[gpu] %s (%d pages, %.2f GB)" % (prob.name, big_pages, big_pages * page_bytes / 1e9))
    o, lse, _ = run_gpu(prob, num_workers=5, dev_inputs=d)
    del big, d
    torch.cuda.empty_cache()
    o, lse = flat(o, lse)
    o_ref, lse_ref = oracle.problem_decode(prob)
    compare(o, lse, o_ref, lse_ref, prob.name)
