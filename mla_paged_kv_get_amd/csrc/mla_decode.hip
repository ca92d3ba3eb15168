// Split-KV decode kernel for MLA over a paged latent cache (gfx950).
//
// What it computes: for each query row, softmax(scale * q K^T) V over the
// attended tokens of its stream, where a token's 576-dim latent is K and its
// first 512 dims are V (FlashMLA source walk-through, data-loading section), and
// the natural log-sum-exp of the scaled scores.  Each worker processes the KV
// tile range the scheduler gave it; a stream handled by one worker gets its
// final o and lse here, otherwise each split leaves a normalised partial o and
// its lse for the combine kernel (same page, scheduling and combine sections).
//
// Mapping to the hardware.  One workgroup (4 waves, one per SIMD) owns 64 query
// rows of one stream; the chip runs one such workgroup per compute unit.  Waves
// 2 r and 2 r + 1 ... are paired as (row block rb = wave & 1, half hf =
// wave >> 1): both waves of a pair own the same 32 rows; the hf wave keeps half
// of the Q dims in VGPRs (dims 256 hf .. + 256 and 512 + 32 hf .. + 32, 18 bf16x8
// fragments) and half of the O^T columns (256 hf .. + 256) in AGPRs.
// Per 32-token sub-tile of the KV stream:
//   1. the page's bf16 rows are staged in a swizzled LDS tile (BF16: direct
//      global->LDS 16-byte loads; FP8: 16-byte loads into VGPRs, e4m3 -> fp32
//      (exact) * scale (RNE) -> bf16 (RNE), then LDS); three buffers keep two
//      sub-tiles in flight behind the one being computed;
//   2. each wave computes its partial S^T = K Q^T over its half of the dims on
//      v_mfma_f32_32x32x16_bf16 (the K tile is the A operand), the pair swaps the
//      partials through LDS and both add them in the same order, so both hold the
//      same scores;
//   3. softmax in the log2 domain, lane-local (S^T puts query row lane % 32 in
//      every lane's accumulator column) against a per-row reference fixed at the
//      first scores of the split (see the main loop), so O and l need no
//      rescaling and O is touched only by MFMAs;
//   4. O^T += V^T P^T on the same MFMA: P goes from the score registers straight
//      into the B operand, V^T comes from the token-major tile through
//      ds_read_b64_tr_b16.
// Tokens that no row attends (page tails, -1 indices) are loaded from a static
// zero token, so every wave issues the same number of loads per sub-tile and
// their scores are masked to -inf.
#include "mla_device.hpp"

namespace mla {

// A token of zeros: the source for slots no query row attends.
__device__ __attribute__((aligned(64))) uint8_t g_zero_token[kBf16TokenBytes] = {0};

namespace {

// Workgroup barrier that orders LDS traffic only.  __syncthreads() implies a
// release fence that also waits for every outstanding global->LDS load, which
// would drain the tiles streaming ahead; these barriers leave them in flight.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Also wait until at most N global->LDS loads of this wave are outstanding:
// with N = the loads one round issues, everything issued before this round has
// landed (the hardware completes these loads in order).
template <int N>
__device__ __forceinline__ void tile_barrier_keep() {
  static_assert(N == 9 || N == 10 || N == 11, "unexpected load count");
  if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 11) asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void tile_barrier_drain() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct buffer loads into LDS: lane i writes 16 (or 4) bytes at dst + 16 i (4 i);
// an offset past the resource's size loads zeros.  (Kept out of lambdas: there
// the builtin makes the host pass drop the kernel.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRefLift = 32.0f;   // log2 units
constexpr float kRefRoom = 88.0f;
constexpr int kSub = 32;                               // tokens per sub-tile
constexpr int kSubBytes = kSub * kBf16TokenBytes;      // 36864
constexpr int kNBuf = 3;
constexpr int kXOffset = kNBuf * kSubBytes;            // S exchange: [4 waves][4][64 lanes] f32x4
constexpr int kXBytes = 4 * 64 * 16 * 4;
// Metadata: BF16 rings int32 ring_idx[8][64], ring_pg[8][64]; FP8 int32
// tokidx[8][32] and uint32 vmask[8] in the same space.
constexpr int kRing = 8;
constexpr int kMetaOffset = kXOffset + kXBytes;
constexpr int kMetaBytes = 2 * kRing * 64 * 4;
constexpr int kFlagOffset = kMetaOffset + kMetaBytes;  // int32 per-wave flags[4]
constexpr int kPOffset = kFlagOffset + 16 * 4;         // P exchange: [2 row blocks][2 k-steps][64 lanes] bf16x8
constexpr int kLdsBytes = kPOffset + 2 * 2 * 64 * 16;
constexpr int kBf16LoadsPerThread = kSubBytes / 16 / kThreads;  // 9
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// FP8 registers of one sub-tile for this thread: token tid / 8, code chunks
// j + 8 i (i = 0..3, j = tid % 8; chunk i uses scale i), the four scales and
// RoPE chunk j.
struct RawFp8 {
  u32x4 v[4];
  u32x4 sc;
  u32x4 r;
};

template <bool FP8, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  MLA_LDS f32x4* xbuf = (MLA_LDS f32x4*)(smem + kXOffset);
  MLA_LDS int32_t* ring_idx = (MLA_LDS int32_t*)(smem + kMetaOffset);
  MLA_LDS int32_t* ring_pg = ring_idx + kRing * 64;
  MLA_LDS int32_t* tokidx = (MLA_LDS int32_t*)(smem + kMetaOffset);
  MLA_LDS uint32_t* vmask = (MLA_LDS uint32_t*)(tokidx + 8 * kSub);
  MLA_LDS int32_t* wflag = (MLA_LDS int32_t*)(smem + kFlagOffset);
  MLA_LDS u32x4* pbuf = (MLA_LDS u32x4*)(smem + kPOffset);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;    // lane half (k-group of the MFMA operands)
  const int l32 = lane & 31;  // query row within the row block
  const int rb = wave & 1;    // row block
  const int hf = wave >> 1;   // half of the dims / columns
  const int partner = wave ^ 2;

  // workgroup -> (worker, row tile); the row tiles of one worker share an XCD
  int w, rt;
  {
    const int g = blockIdx.x;
    if (p.n_rt == 1) {
      w = g;
      rt = 0;
    } else if ((p.W & 7) == 0) {
      const int grp = g / (8 * p.n_rt), rem = g % (8 * p.n_rt);
      rt = rem >> 3;
      w = grp * 8 + (rem & 7);
    } else {
      w = g / p.n_rt;
      rt = g % p.n_rt;
    }
  }
  const int32_t* ent = p.meta + kMetaHeader + (int64_t)w * kSchedStride;
  const int bs = ent[0], bt0 = ent[1], es = ent[2], et = ent[3], split0 = ent[4];
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int32_t* first = p.meta + meta_tile_first(p.W, p.n_streams);
  constexpr int tok_bytes = FP8 ? kFp8TokenBytes : kBf16TokenBytes;

  // ---- per-lane constants -------------------------------------------------------
  // K operand: token l32, chunk c(kk) = 32 hf + 2 kk + h for kk < 16, and
  // 64 + 4 hf + 2 (kk - 16) + h for kk = 16, 17.
  const int ksw = tile_swizzle(l32);
  int kofs[4], kofs_r[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) kofs[m] = l32 * kBf16TokenBytes + 32 * hf * 16 + (((2 * m + h) ^ ksw) << 4);
#pragma unroll
  for (int m = 0; m < 2; ++m) kofs_r[m] = l32 * kBf16TokenBytes + ((64 + ((4 * hf + 2 * m + h) ^ ksw)) << 4);
  // V^T operand (transposed reads): [s2][e4][parity of the column block]
  int vofs[2][2][2];
  {
    const int tl = 4 * h + ((lane & 15) >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const int tok = 16 * s2 + 8 * e4 + tl;
        const int sw = tile_swizzle(tok);
        const int sb = sw >> 2;
        const int base = tok * kBf16TokenBytes + 256 * wave + ((cl ^ (sw & 3)) << 4) + 8 * (lane & 1);
        vofs[s2][e4][0] = base + 64 * sb;
        vofs[s2][e4][1] = base - 64 * sb;
      }
  }
  // BF16 staging: load k of this thread fills LDS slot s = (9 wave + k) 64 + lane,
  // i.e. token dtok[k] of the sub-tile, source chunk dchunk[k]
  // (byte offset doff[k] = dtok[k] * 1152 + 16 * source chunk within the sub-tile)
  int dtok[kBf16LoadsPerThread], dchunk[kBf16LoadsPerThread];
  uint32_t doff[kBf16LoadsPerThread];
#pragma unroll
  for (int k = 0; k < kBf16LoadsPerThread; ++k) {
    const int s = (wave * kBf16LoadsPerThread + k) * 64 + lane;
    dtok[k] = s / kTokenChunks;
    dchunk[k] = (s - dtok[k] * kTokenChunks) ^ tile_swizzle(dtok[k]);
    doff[k] = (uint32_t)(dtok[k] * kBf16TokenBytes + dchunk[k] * 16);
  }
  // exchange slots of this lane: [wave][q4][lane]
  const int xo_base = wave * 4 * 64 + lane, xp_base = partner * 4 * 64 + lane;

  for (int stream = bs; stream <= es && stream < p.n_streams; ++stream) {
    const int ntiles = first[stream + 1] - first[stream];
    const int lo = stream == bs ? bt0 : 0;
    const int hi = stream == es ? et : ntiles;
    if (hi <= lo) continue;
    const int sid = stream == bs ? split0 : split_off[stream];
    const bool final_out = (split_off[stream + 1] - split_off[stream]) == 1;

    const int b = SPARSE ? stream / p.s_q : stream;
    const int64_t row_base = (int64_t)stream * p.R_stream;
    const int seqlen = p.seqlens[b];
    const int32_t* bt_row = p.block_table + (int64_t)b * p.max_blocks;
    const int32_t* idx_row = SPARSE ? p.indices + (int64_t)stream * p.topk : nullptr;
    const __amdgpu_buffer_rsrc_t bt_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)bt_row, 0, p.max_blocks * 4, kBufferFlags);
    // sub-tiles [u0, u1): 32 tokens (dense) or 32 index slots (sparse) each
    const int limit = SPARSE ? p.topk : seqlen;
    const int u0 = 2 * lo;
    const int u1 = min(2 * hi, (limit + kSub - 1) / kSub);

    const int row = rt * 64 + rb * kWaveRows + l32;
    const bool row_ok = row < p.R_stream;

    // Q fragments: dims 256 hf + 16 kk + 8 h (kk < 16), 512 + 32 hf + 16 (kk - 16) + 8 h
    bf16x8 qf[18];
    {
      const uint16_t* qrow = p.q + (row_base + (row_ok ? row : 0)) * kDQK + 8 * h;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const int d = kk < 16 ? 256 * hf + 16 * kk : 512 + 32 * hf + 16 * (kk - 16);
        u32x4 v = *(const u32x4*)(qrow + d);
        if (!row_ok) v = u32x4{0, 0, 0, 0};
        qf[kk] = __builtin_bit_cast(bf16x8, v);
      }
    }

    f32x16 acc[8];

    // ---- per sub-tile metadata ----------------------------------------------------
    // Round u (below) streams sub-tile u + 2 into LDS; whatever it needs to know
    // about a sub-tile (its cache page, or the token rows of its 32 index slots)
    // was fetched rounds ahead into LDS, so no round waits on a load it just issued.
    //
    // BF16 (tiles arrive by direct global->LDS loads): the metadata travels the
    // same way, into rings of 8 sub-tiles, issued at the start of a round and
    // landed by its end.  Round u fetches the page of sub-tile u + 3 (dense), or
    // the indices of sub-tile u + 4 and the pages of sub-tile u + 3's indices
    // (sparse).  No loaded value ever lands in a register inside the loop: the
    // compiler could only wait for such a value by draining every direct load
    // still streaming.
    //
    // FP8 (tiles go through registers): sub-tile u's metadata sits in LDS slot
    // u & 7 (dense: its page; sparse: the token row of each slot, -1 when not
    // attended, and the attended mask); every wave loads the metadata of sub-tile
    // u + 4 during round u and wave 0 publishes it at the end of the round.
    auto slot_ok = [&](int u) { return u < u1 && u * kSub + l32 < p.topk; };  // sparse slot l32 exists
    // BF16 direct metadata loads (64 lanes each; lanes 32..63 repeat 0..31)
    auto meta_dma = [&](int u) {
      if constexpr (SPARSE) {
        // indices of sub-tile u + 4
        const int si = min((u + 4) * kSub + l32, p.topk - 1);
        __builtin_amdgcn_global_load_lds((const void*)(idx_row + si),
                                         (MLA_LDS void*)(ring_idx + ((u + 4) & (kRing - 1)) * 64), 4, 0, 0);
        // pages of sub-tile u + 3's indices
        const int idx = ring_idx[((u + 3) & (kRing - 1)) * 64 + l32];
        const bool ok = slot_ok(u + 3) && idx >= 0;
        __builtin_amdgcn_global_load_lds((const void*)(bt_row + (ok ? idx >> 6 : 0)),
                                         (MLA_LDS void*)(ring_pg + ((u + 3) & (kRing - 1)) * 64), 4, 0, 0);
      } else {
        // page of sub-tile u + 3 (the split's last page past its end)
        buffer_load_lds4(bt_rs, (MLA_LDS void*)(ring_pg + ((u + 3) & (kRing - 1)) * 64),
                         (uint32_t)(min(u + 3, u1 - 1) >> 1) * 4u);
      }
    };
    // BF16 prologue: the same ring entries by plain loads (indices of u0 .. u0 + 3,
    // pages of u0 .. u0 + 2)
    auto meta_fill = [&]() {
      if (wave == 0) {
        if constexpr (SPARSE) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int u = u0 + j;
            const int idx = idx_row[min(u * kSub + l32, p.topk - 1)];
            ring_idx[(u & (kRing - 1)) * 64 + lane] = idx;
            if (j < 3) {
              const bool ok = slot_ok(u) && idx >= 0;
              ring_pg[(u & (kRing - 1)) * 64 + lane] = bt_row[ok ? idx >> 6 : 0];
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const int u = u0 + j;
            ring_pg[(u & (kRing - 1)) * 64 + lane] = bt_row[min(u, u1 - 1) >> 1];
          }
        }
      }
    };
    // FP8 metadata (plain loads)
    auto idx_at = [&](int u) -> int { return slot_ok(u) ? idx_row[u * kSub + l32] : -1; };
    auto tok_of = [&](int idx) -> int {
      const int pg = bt_row[(idx < 0 ? 0 : idx) >> 6];  // always issued
      return idx >= 0 ? pg * kPage + (idx & 63) : -1;
    };
    auto page_load = [&](int u) -> int { return bt_row[min(u, u1 - 1) >> 1]; };
    auto publish = [&](int u, int v) {  // wave 0
      if (SPARSE) {
        const uint64_t m = __ballot(v >= 0);
        if (lane < kSub) tokidx[(u & 7) * kSub + lane] = v;
        if (lane == 0) vmask[u & 7] = (uint32_t)m;
      } else if (lane == 0) {
        tokidx[(u & 7) * kSub] = v;
      }
    };
    // attended mask of sub-tile u's 32 slots (sparse)
    auto sparse_mask = [&](int u) -> uint32_t {
      if constexpr (FP8) {
        return vmask[u & 7];
      } else {
        const bool ok = slot_ok(u) && ring_idx[(u & (kRing - 1)) * 64 + l32] >= 0;
        return (uint32_t)__ballot(ok);
      }
    };
    // ---- staging ------------------------------------------------------------------
    auto buffer = [&](int u) -> MLA_LDS char* { return smem + ((u - u0) % kNBuf) * kSubBytes; };
    // FP8: byte address of stored token t of sub-tile u (the zero token when not attended)
    auto token_ptr = [&](int u, int t) -> const uint8_t* {
      if (SPARSE) {
        const int tok = tokidx[(u & 7) * kSub + t];
        return tok >= 0 ? p.kv + (int64_t)tok * tok_bytes : g_zero_token;
      }
      if (u * kSub + t >= seqlen) return g_zero_token;
      const int page = tokidx[(u & 7) * kSub];
      return p.kv + ((int64_t)page * kPage + (u & 1) * kSub + t) * tok_bytes;
    };
    // BF16 direct loads of sub-tile u: this thread's nine 16-byte pieces.  Dense
    // tiles use buffer loads against the sub-tile's 36,864 bytes, and tokens past
    // the sequence end take an out-of-range offset, which loads zeros; sparse
    // tiles load from per-lane global addresses (the zero token when a slot is
    // not attended).
    struct Bf16Loads {
      __amdgpu_buffer_rsrc_t rs;
      uint32_t voff[kBf16LoadsPerThread];
      const uint8_t* src[kBf16LoadsPerThread];
    };
    auto stage_prep = [&](int u, Bf16Loads& L) {
      const int r = (u & (kRing - 1)) * 64;
      if constexpr (SPARSE) {
        // token row of slot l32, then of each load's token
        const int idx = ring_idx[r + l32];
        const int pg = ring_pg[r + l32];
        const int tok = (slot_ok(u) && idx >= 0) ? pg * kPage + (idx & 63) : -1;
#pragma unroll
        for (int k = 0; k < kBf16LoadsPerThread; ++k) {
          const int tk = __shfl(tok, dtok[k]);
          L.src[k] = (tk >= 0 ? p.kv + (int64_t)tk * kBf16TokenBytes : g_zero_token) + dchunk[k] * 16;
        }
      } else {
        const int page = __builtin_amdgcn_readfirstlane(ring_pg[r]);
        const uint8_t* base = p.kv + ((int64_t)page * kPage + (u & 1) * kSub) * kBf16TokenBytes;
        L.rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, kSubBytes, kBufferFlags);
        if ((u + 1) * kSub <= seqlen) {
#pragma unroll
          for (int k = 0; k < kBf16LoadsPerThread; ++k) L.voff[k] = doff[k];
        } else {
          asm volatile("");  // a real branch: only the last sub-tile pays for this
          const int valid = seqlen - u * kSub;  // tokens of the sub-tile inside the sequence
#pragma unroll
          for (int k = 0; k < kBf16LoadsPerThread; ++k) L.voff[k] = dtok[k] < valid ? doff[k] : (uint32_t)kSubBytes;
        }
      }
    };
    auto stage_issue = [&](const Bf16Loads& L, int k, MLA_LDS char* buf) {
      MLA_LDS void* dst = (MLA_LDS void*)(buf + (wave * kBf16LoadsPerThread + k) * 1024);
      if constexpr (SPARSE)
        __builtin_amdgcn_global_load_lds((const void*)L.src[k], dst, 16, 0, 0);
      else
        buffer_load_lds16(L.rs, dst, L.voff[k]);
    };
    auto stage_bf16 = [&](int u, MLA_LDS char* buf) {
      Bf16Loads L;
      stage_prep(u, L);
#pragma unroll
      for (int k = 0; k < kBf16LoadsPerThread; ++k) stage_issue(L, k, buf);
    };
    auto load_fp8 = [&](int u, RawFp8& r) {
      const int t = tid >> 3, j = tid & 7;
      const uint8_t* pt = token_ptr(u, t);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[i] = *(const u32x4*)(pt + 16 * (j + 8 * i));
      r.sc = *(const u32x4*)(pt + kFp8Dims);
      r.r = *(const u32x4*)(pt + kFp8Dims + 16 + 16 * j);
    };
    auto store_fp8 = [&](const RawFp8& r, MLA_LDS char* buf) {
      const int t = tid >> 3, j = tid & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = j + 8 * i;
        u32x4 lo, hi;
        dequant16(r.v[i], pick_scale(r.sc, i), lo, hi);
        *(MLA_LDS u32x4*)(buf + tile_slot(t, 2 * c) * 16) = lo;
        *(MLA_LDS u32x4*)(buf + tile_slot(t, 2 * c + 1) * 16) = hi;
      }
      *(MLA_LDS u32x4*)(buf + tile_slot(t, 64 + j) * 16) = r.r;
    };
    // ---- score exchange and PV pieces ---------------------------------------------
    // The pair adds its two partial S^T blocks through LDS: slots [wave][q4][lane].
    MLA_LDS f32x4* xo = xbuf + xo_base;
    MLA_LDS f32x4* xp = xbuf + xp_base;
    auto kread = [&](MLA_LDS char* kb, int kk) -> bf16x8 {
      const int off = kk < 16 ? kofs[kk & 3] + (kk >> 2) * 128 : kofs_r[kk - 16];
      return *(MLA_LDS bf16x8*)(kb + off);
    };
    // V^T fragment (this wave's 32-column block cb of its 128 columns, 16-token k-step s2)
    auto vread = [&](MLA_LDS char* vb, int s2, int cb) -> bf16x8 {
      const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + vofs[s2][0][cb & 1] + 64 * cb));
      const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + vofs[s2][1][cb & 1] + 64 * cb));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // Reference maximum m_ref (log2 domain, per row): the row's first finite
    // sub-tile maximum + kRefLift, fixed for the whole split, so P = 2^(x - m_ref)
    // stays within [2^-126, 2^(kRefLift + kRefRoom)] for every score within
    // (kRefRoom, 126 - kRefLift) of that first maximum, and O changes only through
    // MFMAs.  A score more than kRefRoom above m_ref (scores spread by over ~60
    // natural-log units) marks the pass as overflowed and the split is recomputed
    // from the start with the split's true maximum as the reference.
    float m_ref = kNegInf, m_seen = kNegInf, l_sum = 0.f;
    bool redo = false;
    do {
      l_sum = 0.f;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[cb][e] = 0.f;
      if (redo) m_ref = m_seen + kRefLift;
      bool overflow = false;

      // ---- prologue: metadata, sub-tiles u0 and u0 + 1 in LDS, S of u0 ------------
      int idx_pref = -1;  // FP8 sparse: index of slot l32 of sub-tile u + 4
      RawFp8 raw;         // FP8: sub-tile u + 2 in flight in VGPRs
      if constexpr (FP8) {
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = SPARSE ? tok_of(idx_at(u0 + j)) : page_load(u0 + j);
        if (SPARSE) idx_pref = idx_at(u0 + 4);
        if (wave == 0)
#pragma unroll
          for (int j = 0; j < 4; ++j) publish(u0 + j, v[j]);
        __syncthreads();
        load_fp8(u0, raw);
        store_fp8(raw, buffer(u0));
        load_fp8(u0 + 1, raw);
        store_fp8(raw, buffer(u0 + 1));
        load_fp8(u0 + 2, raw);
        __syncthreads();
      } else {
        meta_fill();
        __syncthreads();
        stage_bf16(u0, buffer(u0));
        stage_bf16(u0 + 1, buffer(u0 + 1));
        tile_barrier_drain();
      }
      float x[16];  // full scores S^T of the sub-tile whose softmax comes next
      {
        MLA_LDS char* kb = buffer(u0);
        f32x16 s = {};
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kb, kk), qf[kk], s, 0, 0, 0);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) xo[q4 * 64] = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
        lds_barrier();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 o = xp[q4 * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * q4 + e] = hf == 0 ? s[4 * q4 + e] + o[e] : o[e] + s[4 * q4 + e];
        }
      }

      // One round u: PV of sub-tile u (buffer vb) and QK of sub-tile u + 1 (kb),
      // whose MFMAs run under u's softmax, while sub-tile u + 2 streams into nxt.
      // The buffers are distinct, and saying so (restrict) lets the compiler keep
      // the direct loads in flight across the reads of vb and kb.
      auto round = [&](const int u, MLA_LDS char* __restrict__ vb, MLA_LDS char* __restrict__ kb,
                       MLA_LDS char* __restrict__ nxt) __attribute__((always_inline)) {
        // ---- phase A: metadata, streaming, QK(u + 1) under softmax(u) ---------------
        int meta = 0;  // FP8: metadata of sub-tile u + 4 (published at the end of this round)
        if constexpr (FP8) {
          if (SPARSE) {
            meta = tok_of(idx_pref);
            idx_pref = idx_at(u + 5);
          } else {
            meta = page_load(u + 4);
          }
        } else {
          meta_dma(u);
        }
        __builtin_amdgcn_sched_barrier(0);  // metadata loads stay ahead of the tile loads
        Bf16Loads L;
        if constexpr (FP8) {
          store_fp8(raw, nxt);  // sub-tile u + 2 arrived during the last round
          load_fp8(u + 3, raw);
        } else {
          stage_prep(u + 2, L);
        }
        // mask of sub-tile u: lane holds row l32, tokens 8 (e / 4) + 4 h + e % 4
        const uint32_t tmask = SPARSE ? sparse_mask(u) : 0u;
        const bool full = SPARSE ? tmask == 0xFFFFFFFFu : (u + 1) * kSub <= seqlen;
        if (!full) {
          asm volatile("");  // a real branch: full sub-tiles skip the masking
          const int vcount = seqlen - u * kSub;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int tok = 8 * (e >> 2) + 4 * h + (e & 3);
            const bool ok = SPARSE ? ((tmask >> tok) & 1u) != 0 : tok < vcount;
            x[e] = ok ? x[e] : kNegInf;
          }
        }
        // The issue order is pinned (a scheduling barrier per step): MFMA kk of
        // QK(u + 1), the K fragment six steps ahead, one of the nine tile loads,
        // then a slice of u's softmax.  Softmax: row maximum (log2 domain, the
        // scale is positive), reference update, then P = 2^(scale_log2 S - m_ref)
        // for this wave's k-step (the pair splits the exponentials: the hf wave
        // takes tokens 16 hf .. 16 hf + 15, its x[8 hf ..]).
        constexpr int kAhead = 6;
        bf16x8 kf[18];
#pragma unroll
        for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(kb, kk);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s = {};
        float m4[4], mx = 0.f, msafe = 0.f;
        float xs[8];
        bf16x8 pown;
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
          if (kk + kAhead < 18) kf[kk + kAhead] = kread(kb, kk + kAhead);
          if constexpr (!FP8) {
            if (kk < kBf16LoadsPerThread) stage_issue(L, kk, nxt);
          }
          if (kk < 4) {
            m4[kk] = fmaxf(fmaxf(x[4 * kk], x[4 * kk + 1]), fmaxf(x[4 * kk + 2], x[4 * kk + 3]));
          } else if (kk == 4) {
            mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            // lanes l and l ^ 32 hold the same row (a VALU lane swap, no LDS)
            mx = halves_max(mx) * p.scale_log2;
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[e] = hf == 0 ? x[e] : x[8 + e];
          } else if (kk == 5) {
            m_seen = fmaxf(m_seen, mx);
            if (m_ref == kNegInf && mx != kNegInf) m_ref = mx + kRefLift;
            overflow |= mx > m_ref + kRefRoom;
            msafe = m_ref == kNegInf ? 0.f : m_ref;
          } else if (kk < 14) {
            const int e = kk - 6;
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[e], p.scale_log2, -msafe));
            l_sum += pe;
            pown[e] = (__bf16)pe;
          } else if (kk == 14) {
            pbuf[(rb * 2 + hf) * 64 + lane] = __builtin_bit_cast(u32x4, pown);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();  // every P block of sub-tile u is in LDS

        // ---- phase B: O^T += V^T P^T for sub-tile u ----------------------------------
        const bf16x8 pb0 = __builtin_bit_cast(bf16x8, pbuf[(rb * 2 + 0) * 64 + lane]);
        const bf16x8 pb1 = __builtin_bit_cast(bf16x8, pbuf[(rb * 2 + 1) * 64 + lane]);
        const bf16x8 qb0 = __builtin_bit_cast(bf16x8, pbuf[((rb ^ 1) * 2 + 0) * 64 + lane]);
        const bf16x8 qb1 = __builtin_bit_cast(bf16x8, pbuf[((rb ^ 1) * 2 + 1) * 64 + lane]);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 va[2][4];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) va[s2][cb] = vread(vb, s2, cb);
        __builtin_amdgcn_sched_barrier(0);
        // acc[0..3]: rows of this wave's row block, acc[4..7]: the other row block;
        // columns 128 wave + 32 cb
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][cb], s2 ? pb1 : pb0, acc[cb], 0, 0, 0);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[4 + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][cb], s2 ? qb1 : qb0, acc[4 + cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // the PV MFMAs issue before the round's last waits
        // partial S^T of sub-tile u + 1 to the partner
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) xo[q4 * 64] = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
        if constexpr (FP8) {
          if (wave == 0) publish(u + 4, meta);
          lds_barrier();  // sub-tile u + 2 went through registers
        } else {
          tile_barrier_drain();  // sub-tile u + 2 and the metadata have landed
        }
        // ---- phase C: S of sub-tile u + 1 = (hf 0 partial) + (hf 1 partial) ----------
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 o = xp[q4 * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * q4 + e] = hf == 0 ? s[4 * q4 + e] + o[e] : o[e] + s[4 * q4 + e];
        }
      };
      for (int u = u0; u < u1; ++u) round(u, buffer(u), buffer(u + 1), buffer(u + 2));
      // the last round streamed sub-tiles past the end: let them land before LDS is reused
      tile_barrier_drain();

      // the restart must be taken by the whole workgroup (it contains barriers);
      // the vote is over every lane, so it is taken before the lane-0 store
      const bool wave_overflow = __ballot(overflow) != 0;
      if (lane == 0) wflag[wave] = wave_overflow ? 1 : 0;
      __syncthreads();
      redo = (wflag[0] | wflag[1] | wflag[2] | wflag[3]) != 0;
      __syncthreads();
    } while (redo);

    // ---- epilogue -------------------------------------------------------------------
    // This wave holds O^T for both row blocks (columns 128 wave ..); each row's
    // l and reference come from the pair that owns the row.
    l_sum += __shfl_xor(l_sum, 32);
    {
      // l[row block][k-step][32] (each wave summed its k-step), then m_ref[64]
      MLA_LDS float* lm = (MLA_LDS float*)(smem + kXOffset);
      if (h == 0) {
        lm[(rb * 2 + hf) * 32 + l32] = l_sum;
        if (hf == 0) lm[128 + rb * 32 + l32] = m_ref;
      }
      __syncthreads();
      const float l_own = lm[(rb * 2) * 32 + l32] + lm[(rb * 2 + 1) * 32 + l32];
      const float l_oth = lm[((rb ^ 1) * 2) * 32 + l32] + lm[((rb ^ 1) * 2 + 1) * 32 + l32];
      const float m_oth = lm[128 + (rb ^ 1) * 32 + l32];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float lj = j == 0 ? l_own : l_oth, mj = j == 0 ? m_ref : m_oth;
        const int rowj = rt * 64 + (rb ^ j) * kWaveRows + l32;
        const bool empty = !(lj > 0.f);
        const float inv = empty ? 0.f : 1.f / lj;
        const float lse_v = empty ? kNegInf : (mj + __log2f(lj)) * 0.69314718055994531f;
        if (rowj < p.R_stream) {
          if (final_out) {
            uint16_t* orow = p.o + (row_base + rowj) * kDV + 128 * wave + 4 * h;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const f32x16& a = acc[4 * j + cb];
                bf16x2 v0, v1;
                v0.x = (__bf16)(a[4 * i + 0] * inv);
                v0.y = (__bf16)(a[4 * i + 1] * inv);
                v1.x = (__bf16)(a[4 * i + 2] * inv);
                v1.y = (__bf16)(a[4 * i + 3] * inv);
                *(u32x2*)(orow + cb * 32 + 8 * i) =
                    u32x2{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1)};
              }
            if (j == 0 && h == 0 && hf == 0) p.lse[row_base + rowj] = lse_v;
          } else {
            float* prow = p.part_o + ((int64_t)sid * p.R_stream + rowj) * kDV + 128 * wave + 4 * h;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const f32x16& a = acc[4 * j + cb];
                *(f32x4*)(prow + cb * 32 + 8 * i) =
                    f32x4{a[4 * i] * inv, a[4 * i + 1] * inv, a[4 * i + 2] * inv, a[4 * i + 3] * inv};
              }
            if (j == 0 && h == 0 && hf == 0) p.part_lse[(int64_t)sid * p.R_stream + rowj] = lse_v;
          }
        }
      }
    }
    __syncthreads();  // LDS is reused by the next piece
  }
}

template <bool FP8, bool SPARSE>
hipError_t launch_variant(const DecodeParams& p, hipStream_t stream) {
  static bool attr_set = false;
  auto kern = mla_decode_kernel<FP8, SPARSE>;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.W * p.n_rt), dim3(kThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, bool is_fp8, hipStream_t stream) {
  const bool sparse = p.topk > 0;
  if (is_fp8) return sparse ? launch_variant<true, true>(p, stream) : launch_variant<true, false>(p, stream);
  return sparse ? launch_variant<false, true>(p, stream) : launch_variant<false, false>(p, stream);
}

}  // namespace mla
