"""Pins for the float64 oracle (CPU only).

Each test fixes part of the oracle against something other than itself: values
and layouts the FlashMLA pages print (fixtures under tests/golden/), library
routines (torch's own float8/bf16 conversions, scaled_dot_product_attention,
logsumexp), closed forms and invariants of the definition.  Chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import mla_inputs as mi
import oracle

# --------------------------------------------------------------------------------------
# helpers: an independent widening + attention built from torch library routines


def library_latents(prob):
    """All stored tokens widened to float64 with torch's own conversions: [pool_tokens, 576].

    FP8 dims 0..511 follow the dequantisation the source walk-through describes
    (values turned back into bf16 before the bf16 multiply): torch's fp32
    multiply by the scale, then torch's bf16 cast.
    """
    if prob.is_fp8:
        kv = prob.kvcache.reshape(-1, mi.FP8_TOKEN_BYTES)
        vals = kv[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
        scales = kv[:, 512:528].contiguous().view(torch.float32)
        # dequantised to bf16 before the bf16 multiply: fp32 product, then bf16
        vals = (vals * scales.repeat_interleave(128, dim=1)).to(torch.bfloat16).to(torch.float64)
        rope = kv[:, 528:].contiguous().view(torch.bfloat16).to(torch.float64)
        return torch.cat([vals, rope], dim=1)
    return prob.kvcache.reshape(-1, mi.D_QK).to(torch.float64)


def library_attention(prob, causal=False):
    """o [B, s_q, h_q, 512], lse [B, s_q, h_q] via torch SDPA / logsumexp in float64 (non-empty rows).

    causal (dense): a boolean SDPA mask over the whole sequence, allowing
    position j for query token s when j <= seqlen - s_q + s; rows with no
    allowed position stay NaN."""
    K_all = library_latents(prob)
    B, s_q, h_q = prob.B, prob.s_q, prob.h_q
    o = torch.full((B, s_q, h_q, 512), float("nan"), dtype=torch.float64)
    lse = torch.full((B, s_q, h_q), float("nan"), dtype=torch.float64)
    for b in range(B):
        for s in range(s_q):
            if prob.indices is None:
                pos = torch.arange(int(prob.cache_seqlens[b]))
            else:
                pos = prob.indices[b, s].to(torch.int64)
                pos = pos[pos != -1]
            if pos.numel() == 0:
                continue
            allowed = torch.ones(pos.numel(), dtype=torch.bool)
            if causal:
                allowed = pos <= int(prob.cache_seqlens[b]) - s_q + s
                if not bool(allowed.any()):
                    continue
            phys = prob.block_table[b].to(torch.int64)[pos // 64] * 64 + pos % 64
            K = K_all[phys]
            q = prob.q[b, s].to(torch.float64)
            mask = allowed[None, None, None, :].expand(1, 1, h_q, pos.numel())
            out = F.scaled_dot_product_attention(q[None, None], K[None, None], K[None, None, :, :512].contiguous(),
                                                 attn_mask=mask, scale=prob.softmax_scale)
            o[b, s] = out[0, 0]
            sc = prob.softmax_scale * (q @ K.T)
            lse[b, s] = torch.logsumexp(sc.masked_fill(~allowed[None, :], float("-inf")), dim=-1)
    return o, lse


def run_oracle(prob, rows=None, causal=False):
    o, lse = oracle.problem_decode(prob, rows, causal)
    if rows is None:
        o = o.reshape(prob.B, prob.s_q, prob.h_q, 512)
        lse = lse.reshape(prob.B, prob.s_q, prob.h_q)
    return o, lse


# --------------------------------------------------------------------------------------
# stored-format widening


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_bf16_widening_matches_torch():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(4096, generator=g).to(torch.bfloat16)
    bits = np.concatenate([x.view(torch.int16).numpy().view(np.uint16),
                           np.array([0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0000, 0x8000], dtype=np.uint16)])
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------------------
# the 656-byte token


def test_fp8_token_layout_handbuilt(golden):
    lay = {k: int(v) for k, v in golden("fp8_token_layout.txt").items()}
    assert oracle.token_bytes(True) == lay["token_bytes"] == lay["values_bytes"] + lay["scales_bytes"] + lay["rope_bytes"]
    assert oracle.token_bytes(False) == 2 * lay["latent_dims"]
    tok = np.zeros(lay["token_bytes"], dtype=np.uint8)
    # dim d holds the code d % 127 (all finite codes), so a mis-ordered byte shows
    codes = (np.arange(512) % 127).astype(np.uint8)
    tok[lay["values_offset"]:lay["values_offset"] + 512] = codes
    scales = np.array([1.0, 2.0, 0.25, 3.0], dtype=np.float32)
    tok[lay["scales_offset"]:lay["scales_offset"] + 16] = scales.view(np.uint8)
    rope = (np.arange(64, dtype=np.float32) - 31.5).astype(np.float32)
    rope_bits = torch.from_numpy(rope).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
    tok[lay["rope_offset"]:lay["rope_offset"] + 128] = rope_bits
    k = oracle.token_latent(tok, True)
    e4 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tile = lay["scale_tile_dims"]
    # every code times these scales is exact in bf16, so the decode is exact
    expect = np.concatenate([e4 * np.repeat(scales.astype(np.float64), tile), rope.astype(np.float64)])
    assert np.array_equal(k, expect)


def test_fp8_writer_roundtrip():
    g = torch.Generator().manual_seed(1)
    lat = torch.randn(512, 576, generator=g)
    lat[7, :128] = 0.0  # an all-zero tile
    lat[9, 200] = 1e-3  # subnormal-range element next to larger ones
    toks = mi.quantize_fp8_tokens(lat).numpy()
    assert toks.shape == (512, 656)
    x = lat.numpy().astype(np.float64)
    for t in range(512):
        k = oracle.token_latent(toks[t], True)
        amax = lat[t, :512].reshape(4, 128).abs().amax(dim=1)
        scale = (amax / 448.0).numpy()
        assert np.array_equal(toks[t, 512:528].view(np.float32), scale)  # scales bit-exact at bytes 512..527
        assert np.array_equal(toks[t, 528:656].view(np.uint16),
                              lat[t, 512:].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        for tile in range(4):
            sl = slice(128 * tile, 128 * tile + 128)
            s = float(scale[tile])
            xr, kr = x[t, sl], k[sl]
            if s == 0.0:
                assert np.all(kr == 0.0)
                continue
            # e4m3 rounding (2^-4 relative on normals, scale 2^-10 on subnormals), then bf16 (2^-9)
            normal = np.abs(xr) >= s * 2.0 ** -6
            assert np.all(np.abs(kr - xr)[normal] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(xr)[normal] + 1e-300)
            assert np.all(np.abs(kr - xr)[~normal] <= s * 2.0 ** -10 * (1 + 1e-6) + 2.0 ** -9 * np.abs(kr)[~normal])
            j = int(np.argmax(np.abs(xr)))
            assert abs(abs(kr[j]) - abs(xr[j])) <= 2.0 ** -8 * abs(xr[j])


def test_fp8_dequant_contract_matches_torch():
    codes = np.repeat(np.arange(256, dtype=np.uint8), 6)
    base = np.array([1.0, 0.0023, 3.7e-5, 448.0 / 7.0, 1.5e-38, 2.0 ** -120], dtype=np.float32)
    scales = np.tile(base, 256)
    ours = oracle.fp8_dequant_bf16(codes, scales)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scales)
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(v.numpy())
    assert np.all(((ours[isnan] & 0x7F80) == 0x7F80) & ((ours[isnan] & 0x7F) != 0))
    assert np.array_equal(ours[~isnan], ref[~isnan])


# --------------------------------------------------------------------------------------
# closed forms printed on the pages


def test_cache_size_closed_forms(golden):
    g = golden("cache_sizes.txt")
    tok = oracle.token_bytes(False)
    assert tok == int(g["bf16_token_bytes"])
    total = tok * int(g["layers"]) * int(g["context_tokens"])
    assert total == int(g["bf16_request_bytes_exact"])
    assert round(total / 2 ** 30, 2) == float(g["bf16_request_gib_printed"])
    fp8 = oracle.token_bytes(True) * int(g["layers"]) * int(g["context_tokens"])
    assert 0.5 < fp8 / total < 0.6  # "nearly halves"
    per = int(g["flop_per_row_token"])
    assert per == 2 * (576 + 512)
    assert round(int(g["mma_heads"]) * per / int(g["mma_flop_per_clk"])) == int(g["mma_cycles_printed"])
    prob = mi.make_problem("t", 1, 1, 64, [1], seed=0)
    assert prob.flops() == int(g["mma_heads"]) * per


# --------------------------------------------------------------------------------------
# attention against library routines


CASES = [
    dict(name="dense bf16 ragged", B=3, s_q=2, h_q=4, seqlens=[1, 64, 200], seed=11),
    dict(name="dense fp8", B=2, s_q=1, h_q=3, seqlens=[130, 65], seed=12, is_fp8=True),
    dict(name="sparse bf16 clip", B=2, s_q=2, h_q=4, seqlens=[300, 40], seed=13, topk=70, recipe="clip", n_invalid=5),
    dict(name="sparse fp8", B=2, s_q=1, h_q=4, seqlens=[500, 129], seed=14, topk=100, is_fp8=True, n_invalid=10),
    dict(name="sparse fp8 s_q=2 ragged topk", B=1, s_q=2, h_q=5, seqlens=[1000], seed=15, topk=131, is_fp8=True,
         n_invalid=31),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_matches_library_attention(case):
    c = dict(case)
    prob = mi.make_problem(c.pop("name"), **c)
    o, lse = run_oracle(prob)
    o_ref, lse_ref = library_attention(prob)
    assert np.allclose(o, o_ref.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=1e-12)


def test_duplicate_indices_count_with_multiplicity():
    prob = mi.make_problem("dup", 1, 1, 4, [200], seed=21, topk=8)
    prob.indices[0, 0] = torch.tensor([5, 5, 5, 130, 7, -1, 130, 199], dtype=torch.int32)
    o, lse = run_oracle(prob)
    o_ref, lse_ref = library_attention(prob)  # gathers K with repeats, so multiplicity counts
    assert np.allclose(o, o_ref.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------
# closed forms and special cases of the definition


@pytest.mark.parametrize("is_fp8", [False, True])
def test_uniform_scores_give_mean_of_v(is_fp8):
    prob = mi.make_problem("q0", 2, 1, 2, [4096, 77], seed=31, is_fp8=is_fp8, q_zero=True)
    o, lse = run_oracle(prob)
    K = library_latents(prob).numpy()
    for b, L in enumerate([4096, 77]):
        pos = np.arange(L)
        phys = prob.block_table[b].numpy()[pos // 64] * 64 + pos % 64
        mean = K[phys, :512].mean(axis=0)
        assert np.allclose(o[b, 0], mean, rtol=0, atol=1e-13)
        assert np.allclose(lse[b, 0], math.log(L), rtol=0, atol=1e-13)
    assert abs(lse[0, 0, 0] - 8.317766166719343) < 1e-12  # ln 4096


def test_empty_attended_set():
    prob = mi.make_problem("empty", 2, 2, 3, [0, 50], seed=41)
    o, lse = run_oracle(prob)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    sp = mi.make_problem("all -1", 2, 1, 3, [100, 100], seed=42, topk=64)
    sp.indices[1] = -1
    o, lse = run_oracle(sp)
    assert np.all(o[1] == 0.0) and np.all(lse[1] == -np.inf)
    assert np.all(np.isfinite(lse[0]))


@pytest.mark.parametrize("is_fp8", [False, True])
def test_single_token_returns_its_v(is_fp8):
    prob = mi.make_problem("one", 1, 1, 3, [300], seed=51, topk=64, is_fp8=is_fp8)
    prob.indices[0, 0] = -1
    prob.indices[0, 0, 17] = 233
    o, lse = run_oracle(prob)
    K = library_latents(prob).numpy()
    phys = int(prob.block_table[0, 233 // 64]) * 64 + 233 % 64
    for h in range(3):
        assert np.array_equal(o[0, 0, h], K[phys, :512])
        q = prob.q[0, 0, h].to(torch.float64).numpy()
        assert abs(lse[0, 0, h] - prob.softmax_scale * float(q @ K[phys])) < 1e-12


def test_split_invariance():
    """Any partition of the attended set, merged by lse, equals the unsplit result."""
    prob = mi.make_problem("split", 1, 1, 2, [777], seed=61, is_fp8=True)
    q = prob.q.view(torch.int16).numpy().view(np.uint16)
    kv = prob.kvcache.view(torch.uint8).numpy()
    bt = prob.block_table[0].numpy()
    pos = np.arange(777)
    rng = np.random.default_rng(0)
    for h in range(2):
        o_full, lse_full = oracle.attend(q[0, 0, h], kv, True, bt, pos, prob.softmax_scale)
        for trial in range(6):
            if trial < 3:  # contiguous pieces, some empty
                cuts = np.sort(rng.integers(0, 778, size=trial + 3))
                parts = np.split(pos, cuts)
            else:  # arbitrary subsets
                lab = rng.integers(0, trial + 1, size=777)
                parts = [pos[lab == i] for i in range(trial + 2)]  # the last part is empty
            res = [oracle.attend(q[0, 0, h], kv, True, bt, p, prob.softmax_scale) for p in parts]
            o, lse = oracle.lse_combine(np.stack([r[0] for r in res]), np.array([r[1] for r in res]))
            assert np.allclose(o, o_full, rtol=1e-12, atol=1e-13)
            assert abs(lse - lse_full) < 1e-12
    o, lse = oracle.lse_combine(np.zeros((3, 512)), np.full(3, -np.inf))
    assert np.all(o == 0.0) and lse == -np.inf


def test_dense_equals_sparse_with_full_index_list():
    dense = mi.make_problem("d", 2, 2, 3, [150, 64], seed=71)
    sparse = mi.make_problem("d", 2, 2, 3, [150, 64], seed=71)
    topk = 192
    idx = torch.full((2, 2, topk), -1, dtype=torch.int32)
    for b, L in enumerate([150, 64]):
        idx[b, :, :L] = torch.arange(L, dtype=torch.int32)
    sparse.indices = idx
    od, ld = run_oracle(dense)
    os_, ls = run_oracle(sparse)
    assert np.array_equal(od, os_) and np.array_equal(ld, ls)


def test_page_permutation_invariance():
    prob = mi.make_problem("perm", 2, 1, 4, [200, 90], seed=81, n_spare=3)
    o1, l1 = run_oracle(prob)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(prob.num_blocks, generator=g)  # new slot of old page p is inv[p]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    prob.kvcache = prob.kvcache[perm].contiguous()
    prob.block_table = inv[prob.block_table.to(torch.int64)].to(torch.int32)
    o2, l2 = run_oracle(prob)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8_equals_bf16_on_representable_data():
    """Latents that are e4m3 codes times power-of-two scales (amax at 448) decode
    identically from the FP8 and BF16 caches."""
    gen = torch.Generator().manual_seed(91)
    n_pages = 6  # ceil(256/64) + ceil(100/64)
    n = n_pages * 64
    codes = torch.randint(0, 256, (n, 512), generator=gen, dtype=torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
    codes[:, ::128] = 0x7E  # each tile reaches 448
    exps = torch.randint(-6, 3, (n, 4), generator=gen)
    scales = torch.pow(2.0, exps.to(torch.float32))
    rope = torch.randn(n, 64, generator=gen).to(torch.bfloat16)
    fp8 = torch.cat([codes, scales.view(torch.uint8).reshape(n, 16), rope.view(torch.uint8).reshape(n, 128)], dim=1)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float32) * scales.repeat_interleave(128, dim=1)
    bf = torch.cat([vals.to(torch.bfloat16), rope], dim=1)
    assert torch.equal(bf[:, :512].to(torch.float32), vals)  # representable
    p8 = mi.make_problem("fp8", 2, 1, 4, [256, 100], seed=92, n_spare=0, is_fp8=True)
    pb = mi.make_problem("fp8", 2, 1, 4, [256, 100], seed=92, n_spare=0)
    assert p8.num_blocks == n_pages
    p8.kvcache = fp8.view(n_pages, 64, 656).contiguous()
    pb.kvcache = bf.view(n_pages, 64, 576).contiguous()
    o8, l8 = run_oracle(p8)
    ob, lb = run_oracle(pb)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def exact_product_attention(prob):
    """o, lse of the FP8 problem with each element read as the exact product
    e4m3fn(code) x scale in float64 (no rounding to fp32 or bf16), via torch
    SDPA / logsumexp in float64: the other reading of the dequantisation."""
    kv = prob.kvcache.reshape(-1, mi.FP8_TOKEN_BYTES)
    vals = kv[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    scales = kv[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
    rope = kv[:, 528:].contiguous().view(torch.bfloat16).to(torch.float64)
    K_all = torch.cat([vals * scales.repeat_interleave(128, dim=1), rope], dim=1)
    o = np.full((prob.B * prob.s_q * prob.h_q, 512), np.nan)
    lse = np.full(prob.B * prob.s_q * prob.h_q, np.nan)
    for b in range(prob.B):
        for s in range(prob.s_q):
            pos = prob.indices[b, s].to(torch.int64)
            pos = pos[pos != -1]
            phys = prob.block_table[b].to(torch.int64)[pos // 64] * 64 + pos % 64
            K = K_all[phys]
            q = prob.q[b, s].to(torch.float64)
            r = (b * prob.s_q + s) * prob.h_q
            o[r:r + prob.h_q] = F.scaled_dot_product_attention(
                q[None, None], K[None, None], K[None, None, :, :512].contiguous(), scale=prob.softmax_scale)[0, 0].numpy()
            lse[r:r + prob.h_q] = torch.logsumexp(prob.softmax_scale * (q @ K.T), dim=-1).numpy()
    return o, lse


@pytest.mark.parametrize("recipe", ["c4", "c5"])
def test_fp8_bf16_reading_within_tolerance_of_exact_product(recipe):
    """The oracle reads an FP8 element as bf16(fp32(code x scale)) (the kernel
    turns the values back into bf16 before its bf16 multiply); the exact product
    code x scale is the other plain reading.  On inputs made like the sparse FP8
    workloads (random latents quantised per 128-dim tile, index lists with -1
    slots) the two readings differ by a small part of the parity tolerance
    (measured: o by 5-7 % of its bound, lse by 1.6e-4-2.6e-4 against 1e-3), so
    the choice between them cannot decide a parity result."""
    if recipe == "c4":
        prob = mi.make_problem("fp8 reading", 3, 1, 128, [32768, 20000, 5000], seed=501, topk=2048, is_fp8=True,
                               n_invalid=102)
    else:
        prob = mi.make_problem("fp8 reading", 2, 2, 64, [8192, 1024], seed=502, topk=2048, is_fp8=True,
                               n_invalid=0, recipe="clip")
    o_b, l_b = oracle.problem_decode(prob)
    o_x, l_x = exact_product_attention(prob)
    do = np.abs(o_b - o_x)
    ratio = (do / (8e-3 + 1e-2 * np.abs(o_x))).max()
    dl = np.abs(l_b - l_x).max()
    # the bf16 step moves each element by at most 2^-9 of itself, and a score
    # (a sum over 576 products) by less; o and lse stay well inside
    # |d o| <= 8e-3 + 1e-2 |o| and |d lse| <= 1e-3
    assert ratio < 0.1, ratio
    assert dl < 0.5e-3, dl
    assert do.max() > 0.0  # the readings do differ: the bf16 step is not a no-op here


@pytest.mark.parametrize("is_fp8,topk", [(False, 0), (True, 96)])
def test_unattended_tokens_are_never_read(is_fp8, topk):
    kw = dict(B=2, s_q=1, h_q=3, seqlens=[130, 70], seed=101, is_fp8=is_fp8, topk=topk, n_spare=2, max_blocks=4)
    if topk:
        kw["recipe"] = "clip"
    clean = mi.make_problem("clean", **kw)
    dirty = mi.make_problem("dirty", nan_fill=True, **kw)
    assert not torch.equal(clean.kvcache.view(torch.uint8), dirty.kvcache.view(torch.uint8))
    o1, l1 = run_oracle(clean)
    o2, l2 = run_oracle(dirty)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full():
    prob = mi.make_problem("rows", 2, 2, 3, [90, 200], seed=111)
    o, lse = oracle.problem_decode(prob)
    rows = np.array([11, 0, 5, 5, 7])
    o2, l2 = oracle.problem_decode(prob, rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(l2, lse[rows])


# --------------------------------------------------------------------------------------
# the schedule rule (this project's own design): coverage and balance


def _walk(sched, off, tiles, q, n_workers):
    n_streams = len(tiles)
    seen = [np.zeros(t, dtype=np.int64) for t in tiles]
    split_owner = {}
    for w in range(n_workers):
        bs, bt, es, et, first = sched[w, :5]
        if bs == es and bt == et:
            continue
        count = 0
        sid = first
        for i in range(bs, min(es, n_streams - 1) + 1):
            lo = bt if i == bs else 0
            hi = et if i == es else tiles[i]
            if hi <= lo:
                continue
            seen[i][lo:hi] += 1
            count += hi - lo
            if i != bs:
                sid = off[i]
            assert off[i] <= sid < off[i + 1]
            assert sid not in split_owner
            split_owner[sid] = (w, i)
        assert count <= q
    for i in range(n_streams):
        assert np.all(seen[i] == 1)
    assert sorted(split_owner) == list(range(off[-1]))


@pytest.mark.parametrize("seed", range(6))
def test_schedule_covers_every_tile_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    s_q = int(rng.integers(1, 3))
    topk = int(rng.choice([0, 0, 64, 100, 2048]))
    seqlens = rng.integers(0, 5000, size=B).astype(np.int32)
    seqlens[rng.random(B) < 0.2] = 0
    W = int(rng.choice([1, 7, 64, 256, 1000]))
    min_tiles = int(rng.choice([1, 2, 4, 16]))
    sched, off = oracle.schedule(seqlens, s_q, topk, W, min_tiles)
    tiles = [(-(-topk // 64)) for _ in range(B * s_q)] if topk else [int(-(-s // 64)) for s in seqlens]
    N = sum(tiles)
    q = max(-(-N // W), min_tiles, 1)
    _walk(sched, off, tiles, q, W)
    busy = sum(1 for w in range(W) if not (sched[w, 0] == sched[w, 2] and sched[w, 1] == sched[w, 3]))
    assert busy == min(W, -(-N // q)) if N else busy == 0


# --------------------------------------------------------------------------------------
# causal masking (speculative decoding, s_q > 1): the usage example on the geoz.com.cn
# page passes causal=True; the mask is aligned to the end of the cache, so query token
# s of s_q sees positions j <= seqlen - s_q + s


CAUSAL_CASES = [
    dict(name="bf16 s_q=3 short and ragged", B=4, s_q=3, h_q=4, seqlens=[1, 2, 64, 200], seed=81),
    dict(name="fp8 s_q=4", B=2, s_q=4, h_q=3, seqlens=[130, 5], seed=82, is_fp8=True),
    dict(name="bf16 s_q=2 page edge", B=2, s_q=2, h_q=2, seqlens=[65, 128], seed=83),
]


@pytest.mark.parametrize("case", CAUSAL_CASES, ids=[c["name"] for c in CAUSAL_CASES])
def test_causal_matches_library_attention(case):
    c = dict(case)
    prob = mi.make_problem(c.pop("name"), **c)
    o, lse = run_oracle(prob, causal=True)
    o_ref, lse_ref = library_attention(prob, causal=True)
    for b, L in enumerate(c["seqlens"]):
        for s in range(prob.s_q):
            if L - prob.s_q + s < 0:  # the query token sees nothing
                assert np.all(o[b, s] == 0.0) and np.all(lse[b, s] == -np.inf)
            else:
                assert np.allclose(o[b, s], o_ref[b, s].numpy(), rtol=1e-11, atol=1e-12)
                assert np.allclose(lse[b, s], lse_ref[b, s].numpy(), rtol=1e-12, atol=1e-12)


def test_causal_uniform_scores_give_prefix_mean():
    L, s_q = 300, 4
    prob = mi.make_problem("cq0", 1, s_q, 2, [L], seed=84, q_zero=True)
    o, lse = run_oracle(prob, causal=True)
    K = library_latents(prob).numpy()
    for s in range(s_q):
        n = L - s_q + s + 1
        pos = np.arange(n)
        phys = prob.block_table[0].numpy()[pos // 64] * 64 + pos % 64
        assert np.allclose(o[0, s], K[phys, :512].mean(axis=0), rtol=0, atol=1e-13)
        assert np.allclose(lse[0, s], math.log(n), rtol=0, atol=1e-13)


def test_causal_with_one_query_token_is_the_full_sequence():
    prob = mi.make_problem("c1", 3, 1, 4, [1, 77, 640], seed=85)
    oc, lc = run_oracle(prob, causal=True)
    on, ln = run_oracle(prob)
    assert np.array_equal(oc, on) and np.array_equal(lc, ln)


def test_causal_rejects_sparse():
    prob = mi.make_problem("cs", 1, 2, 2, [100], seed=86, topk=16)
    with pytest.raises(ValueError):
        run_oracle(prob, causal=True)


def test_sparse_prefill_problem_is_plain_gather_attention():
    """A sparse prefill problem (one contiguous KV sequence, identity page table)
    reaches the oracle as a one-request sparse decode; its result must equal
    attention written directly on the contiguous rows: for query token s, the
    rows kv[indices[s]] (-1 dropped) as K, their first 512 dims as V, in float64."""
    prob = mi.make_prefill_problem("prefill pin", 6, 3, 150, 40, seed=17, n_invalid=7, recipe="clip")
    o, lse = run_oracle(prob)
    o = o.reshape(6, 3, 512)
    lse = lse.reshape(6, 3)
    kv = prob.kvcache.reshape(-1, 576)[:150].double()
    q = prob.q[0].double()
    for s in range(6):
        rows = prob.indices[0, s].long()
        rows = rows[rows >= 0]
        k = kv[rows]
        for h in range(3):
            logits = prob.softmax_scale * (k @ q[s, h])
            m = logits.max()
            w = torch.exp(logits - m)
            ref_o = (w[:, None] * k[:, :512]).sum(0) / w.sum()
            ref_lse = float(m + torch.log(w.sum()))
            assert np.allclose(o[s, h], ref_o.numpy(), rtol=1e-11, atol=1e-12)
            assert abs(lse[s, h] - ref_lse) < 1e-11
