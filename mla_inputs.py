"""Seeded synthetic inputs for MLA decoding over a paged latent KV cache.

This module only builds input bytes; it holds none of the decode arithmetic.  It
is shared by the tests, the oracle checks and the benchmark, and it imports
neither the oracle nor the GPU package.

Shapes follow the FlashMLA pages: a query is [B, s_q, h_q, 576] bf16; one KV
head whose 576-dim latent per token serves as K (its first 512 dims as V); the
cache is paged in 64-token blocks addressed through block_table[B, max_blocks]
with cache_seqlens[B] tokens per request; sparse decoding passes
indices[B, s_q, topk] int32 with -1 entries ignored.  The FP8 cache stores a
token in 656 bytes: 512 OCP e4m3fn codes (byte d = dim d), four little-endian
fp32 scales (scale t covers dims [128 t, 128 t + 128)), then the 64 RoPE dims as
little-endian bf16.

Writing the FP8 cache is the cache writer's job, not the decoder's; the writer
here follows the 1x128 tile quantisation the source walk-through describes:
scale = fp32(amax / 448), code = round-to-nearest-even of
clamp(x / scale, -448, 448) in e4m3fn (torch's cast), code 0 for an all-zero
tile.  The clamp matters: torch's cast returns NaN above 448 instead of
saturating.

Draw order inside one problem (one torch CPU generator): sequence lengths ->
page permutation -> q -> latents -> indices.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

PAGE = 64
D_QK = 576
D_V = 512
FP8_DIMS = 512
FP8_TOKEN_BYTES = 656
BF16_TOKEN_BYTES = 1152
_LATENT_CHUNK = 1 << 16  # tokens per randn call; fixed so the stream is reproducible


@dataclass
class Problem:
    """One decode call's inputs, all on the CPU."""

    name: str
    q: torch.Tensor  # bf16 [B, s_q, h_q, 576]
    kvcache: torch.Tensor  # bf16 [num_blocks, 64, 576] or uint8 [num_blocks, 64, 656]
    block_table: torch.Tensor  # int32 [B, max_blocks]
    cache_seqlens: torch.Tensor  # int32 [B]
    indices: Optional[torch.Tensor]  # int32 [B, s_q, topk] or None (dense)
    is_fp8: bool
    softmax_scale: float
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def topk(self) -> int:
        return 0 if self.indices is None else int(self.indices.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.kvcache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def attended_tokens(self) -> int:
        """Number of (query token, attended KV token) pairs summed over requests.

        Dense: every query token of request b attends seqlen_b tokens.  Sparse:
        each (b, s) attends its non-(-1) indices.
        """
        if self.indices is None:
            return int(self.cache_seqlens.to(torch.int64).sum().item()) * self.s_q
        return int((self.indices != -1).sum().item())

    def flops(self) -> float:
        """2 * (576 + 512) FLOP per query row per attended token."""
        return 2.0 * (D_QK + D_V) * self.h_q * self.attended_tokens()

    def bytes(self) -> float:
        """Attended KV bytes plus q and o bytes.

        Dense: each request's KV is read once for all its query rows.  Sparse:
        every attended index is a separate token read.
        """
        tok = FP8_TOKEN_BYTES if self.is_fp8 else BF16_TOKEN_BYTES
        if self.indices is None:
            kv = int(self.cache_seqlens.to(torch.int64).sum().item()) * tok
        else:
            kv = self.attended_tokens() * tok
        rows = self.B * self.s_q * self.h_q
        return float(kv + rows * D_QK * 2 + rows * D_V * 2)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """The raw 16-bit patterns of a bf16 tensor (as int16)."""
    return t.contiguous().view(torch.int16)


def quantize_fp8_tokens(lat: torch.Tensor) -> torch.Tensor:
    """fp32 latents [n, 576] -> 656-byte FP8 tokens [n, 656] (uint8)."""
    lat = lat.to(torch.float32)
    n = lat.shape[0]
    x = lat[:, :FP8_DIMS].reshape(n, 4, 128)
    amax = x.abs().amax(dim=-1)
    scale = amax / 448.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = x / safe[..., None]
    y = torch.where(scale[..., None] > 0, y, torch.zeros_like(y))
    codes = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, FP8_DIMS)
    sc = scale.contiguous().view(torch.uint8).reshape(n, 16)
    rope = lat[:, FP8_DIMS:].to(torch.bfloat16).contiguous().view(torch.uint8).reshape(n, 128)
    return torch.cat([codes, sc, rope], dim=1).contiguous()


def _fill_cache(gen: torch.Generator, num_blocks: int, is_fp8: bool) -> torch.Tensor:
    """Pool of num_blocks pages of N(0,1) latents, written as bf16 or FP8 tokens."""
    n_tokens = num_blocks * PAGE
    width = FP8_TOKEN_BYTES if is_fp8 else D_QK
    out = torch.empty((n_tokens, width), dtype=torch.uint8 if is_fp8 else torch.bfloat16)
    for lo in range(0, n_tokens, _LATENT_CHUNK):
        hi = min(n_tokens, lo + _LATENT_CHUNK)
        lat = torch.randn((hi - lo, D_QK), generator=gen, dtype=torch.float32)
        out[lo:hi] = quantize_fp8_tokens(lat) if is_fp8 else lat.to(torch.bfloat16)
    return out.view(num_blocks, PAGE, width)


def _page_layout(gen: torch.Generator, seqlens: Sequence[int], n_spare: int, max_blocks: Optional[int]):
    """Shuffled page pool: request b gets the next ceil(seqlen_b/64) entries of a
    random permutation of the pool, in request order; the last n_spare entries
    are spare pages and fill unused block_table entries."""
    need = [(int(s) + PAGE - 1) // PAGE for s in seqlens]
    pool = sum(need) + n_spare
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    width = max(max(need) if need else 0, 1) if max_blocks is None else max_blocks
    fill = int(perm[pool - 1]) if n_spare > 0 else 0
    bt = torch.full((len(seqlens), width), fill, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, pool


def _sparse_indices(gen: torch.Generator, seqlens: Sequence[int], s_q: int, topk: int, n_invalid: int,
                    recipe: str) -> torch.Tensor:
    """indices[B, s_q, topk]: positions drawn without replacement from [0, seqlen_b).

    recipe "sample": the first topk of a random permutation of [0, seqlen_b)
    (seqlen_b >= topk), then n_invalid random slots set to -1.
    recipe "clip": as "sample" when seqlen_b >= topk; otherwise a random
    permutation of all seqlen_b positions followed by -1 padding.
    """
    B = len(seqlens)
    idx = torch.full((B, s_q, topk), -1, dtype=torch.int32)
    for b in range(B):
        L = int(seqlens[b])
        for s in range(s_q):
            perm = torch.randperm(L, generator=gen).to(torch.int32)
            if L >= topk:
                idx[b, s] = perm[:topk]
            else:
                if recipe != "clip":
                    raise ValueError("seqlen shorter than topk needs the 'clip' recipe")
                idx[b, s, :L] = perm
            if n_invalid > 0:
                slots = torch.randperm(topk, generator=gen)[:n_invalid]
                idx[b, s, slots] = -1
    return idx


def make_problem(name: str, B: int, s_q: int, h_q: int, seqlens: Sequence[int], *, seed: int, topk: int = 0,
                 is_fp8: bool = False, n_invalid: int = 0, recipe: str = "sample", n_spare: int = 1,
                 max_blocks: Optional[int] = None, softmax_scale: Optional[float] = None,
                 nan_fill: bool = False, q_zero: bool = False) -> Problem:
    """Build one seeded problem.  seqlens may be a list or a callable(gen) -> list."""
    gen = torch.Generator().manual_seed(seed)
    if callable(seqlens):
        seqlens = seqlens(gen)
    seqlens = [int(s) for s in seqlens]
    if len(seqlens) != B:
        raise ValueError("need one seqlen per request")
    bt, pool = _page_layout(gen, seqlens, n_spare, max_blocks)
    q = torch.randn((B, s_q, h_q, D_QK), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    if q_zero:
        q.zero_()
    kv = _fill_cache(gen, pool, is_fp8)
    indices = _sparse_indices(gen, seqlens, s_q, topk, n_invalid, recipe) if topk > 0 else None
    prob = Problem(name=name, q=q, kvcache=kv, block_table=bt,
                   cache_seqlens=torch.tensor(seqlens, dtype=torch.int32), indices=indices, is_fp8=is_fp8,
                   softmax_scale=float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D_QK)),
                   meta=dict(seed=seed, recipe=recipe, n_invalid=n_invalid, n_spare=n_spare))
    if nan_fill:
        poison_unattended(prob)
    return prob


def make_prefill_problem(name: str, s_q: int, h_q: int, s_kv: int, topk: int, *, seed: int, n_invalid: int = 0,
                         recipe: str = "sample") -> Problem:
    """A sparse prefill call as a one-request problem: one contiguous KV sequence
    of s_kv tokens (N(0,1) latents in bf16), whose pages are its consecutive
    64-token pieces (identity block table), and s_q query tokens with their own
    topk index lists.  The prefill call reads kvcache.view(-1, 576)[:s_kv], q[0]
    and indices[0]."""
    gen = torch.Generator().manual_seed(seed)
    n_pages = (int(s_kv) + PAGE - 1) // PAGE
    q = torch.randn((1, s_q, h_q, D_QK), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    kv = _fill_cache(gen, n_pages, False)
    indices = _sparse_indices(gen, [int(s_kv)], s_q, topk, n_invalid, recipe)
    return Problem(name=name, q=q, kvcache=kv, block_table=torch.arange(n_pages, dtype=torch.int32).view(1, -1),
                   cache_seqlens=torch.tensor([int(s_kv)], dtype=torch.int32), indices=indices, is_fp8=False,
                   softmax_scale=1.0 / math.sqrt(D_QK), meta=dict(seed=seed, recipe=recipe, n_invalid=n_invalid))


def attended_mask(prob: Problem) -> torch.Tensor:
    """bool [num_blocks, 64]: which stored tokens any query row can reach."""
    mask = torch.zeros((prob.num_blocks, PAGE), dtype=torch.bool)
    for b in range(prob.B):
        L = int(prob.cache_seqlens[b])
        if prob.indices is None:
            pos = torch.arange(L)
        else:
            pos = prob.indices[b].reshape(-1).to(torch.int64)
            pos = pos[pos != -1]
        pages = prob.block_table[b].to(torch.int64)[pos // PAGE]
        mask[pages, pos % PAGE] = True
    return mask


def poison_unattended(prob: Problem) -> None:
    """Overwrite every unreachable stored token with NaN bytes (bf16 NaN; for FP8
    the NaN code 0x7F, NaN scales and NaN RoPE)."""
    dead = ~attended_mask(prob)
    if prob.is_fp8:
        tok = torch.empty(FP8_TOKEN_BYTES, dtype=torch.uint8)
        tok[:FP8_DIMS] = 0x7F
        tok[FP8_DIMS:FP8_DIMS + 16] = torch.tensor([float("nan")] * 4, dtype=torch.float32).view(torch.uint8)
        tok[FP8_DIMS + 16:] = torch.full((64,), float("nan"), dtype=torch.bfloat16).view(torch.uint8)
        prob.kvcache[dead] = tok
    else:
        prob.kvcache[dead] = float("nan")


# ---- the five standard workloads ---------------------------------------------

def _c3_seqlens(gen: torch.Generator) -> List[int]:
    u = torch.randint(1024, 32768 + 1, (128,), generator=gen)
    s = ((u + 32) // 64) * 64
    return s.clamp(1024, 32768).tolist()


CONFIGS = {
    1: dict(name="tiny dense bf16 (B=2, h_q=16, seqlens {64,200})", B=2, s_q=1, h_q=16, seqlens=[64, 200],
            n_spare=1, max_blocks=4),
    2: dict(name="dense bf16 memory-bound (B=64, h_q=128, seqlen 4096)", B=64, s_q=1, h_q=128,
            seqlens=[4096] * 64, n_spare=0),
    3: dict(name="dense bf16 compute-bound (B=128, s_q=2, h_q=128, seqlen U[1024,32768])", B=128, s_q=2, h_q=128,
            seqlens=_c3_seqlens, n_spare=1, max_blocks=512),
    4: dict(name="sparse fp8 (B=64, h_q=128, seqlen 32768, topk 2048, 5% -1)", B=64, s_q=1, h_q=128,
            seqlens=[32768] * 64, n_spare=0, topk=2048, is_fp8=True, n_invalid=102),
    5: dict(name="skewed sparse fp8 (B=8, s_q=2, h_q=64, seqlens {131072, 1024x7}, topk 2048)", B=8, s_q=2,
            h_q=64, seqlens=[131072] + [1024] * 7, n_spare=1, max_blocks=2048, topk=2048, is_fp8=True,
            recipe="clip"),
}


def config(i: int, *, nan_fill: bool = False) -> Problem:
    """Standard workload i (1..5), seeded with seed = i."""
    c = dict(CONFIGS[i])
    name = c.pop("name")
    return make_problem(name, seed=i, nan_fill=nan_fill, **c)
