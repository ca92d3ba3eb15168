// Split-KV decode kernel for the FP8 (656-byte token) caches, dense and sparse,
// with specialised waves (gfx950).
//
// What it computes is what the general decode kernel computes: for each query
// row, softmax(scale * q K^T) V over the tokens the row attends, a token's
// 576-dim latent being K and its first 512 dims V (FlashMLA source walk-through,
// data-loading section), and the natural log-sum-exp of the scaled scores, with
// the FP8 token decoded as bf16(fp32(e4m3 code) * scale of its 128-dim tile) for
// the 512 coded dims and its 64 bf16 RoPE dims as they are (same page, the
// 656-byte layout).  A stream handled by one worker gets its final o and lse,
// otherwise each split leaves a normalised partial o and its lse for the combine
// kernel (same page, scheduling and combine sections).  Sparse: token slot i of
// a query token's index list names cache position indices[i], -1 = not attended.
//
// Mapping: one workgroup of 8 waves owns 64 query rows of one stream and walks
// its slot (sparse) or token (dense) range in 32-entry sub-tiles, as the dense
// BF16 kernel does.  Waves w and w + 4 share a SIMD and take different roles:
//  - score waves 0..3: S^T for rows 32 (w / 2) .. + 31 and tokens 16 (w % 2) ..
//    + 15 of each sub-tile (each K fragment read from LDS feeds two MFMAs), the
//    softmax and the bf16 P blocks;
//  - PV waves 4..7: wave 4 + c owns O columns 128 c .. 128 c + 127 for all 64 rows.
// Every wave decodes 4 tokens of each sub-tile (tokens 8 k + w): their codes,
// scales and RoPE bytes go into VGPRs one round before the wave writes them as
// bf16 into the swizzled LDS tile, so the dequantising VALU work is spread over
// all 8 waves (staging by the PV waves alone made them the bottleneck: c4 +15 %;
// three of the score wave's four tokens, or two, and the rest by the PV waves:
// +8 % and +13 %).  A wave issues about one VALU instruction every 7 clocks
// (two waves of a SIMD at that rate each), so each wave's VALU count per round
// is kept down: per-lane offsets stay in registers, the metadata is the PV
// waves' work, and the sparse mask is computed once for both row blocks.
// Round u (one barrier): the score waves compute S and P of sub-tile u, the PV
// waves P V of sub-tile u - 1 and V^T of sub-tile u, and every wave writes its
// share of sub-tile u + 2 (loaded in round u - 1) and loads its share of
// sub-tile u + 3.  A wave's LDS operations complete in order, so the ring reads
// a round needs are issued at its start, ahead of the wave's tile writes (c4
// -4 %); writing a score wave's share after its last K read instead of after
// its first MFMA pair measured the same.
#include "mla_device.hpp"

namespace mla {
namespace {

constexpr int kThreads8 = 512;  // 8 waves
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRefLift = 32.0f;  // log2 units
constexpr float kRefRoom = 88.0f;
constexpr int kSub = 32;                           // tokens (slots) per sub-tile
constexpr int kSubBytes = kSub * kBf16TokenBytes;  // 36864: the decoded bf16 tile
constexpr int kNBuf = 4;
// P exchange: [2 (sub-tile parity)][2 row blocks of 32][2 k-steps of 16 tokens][64 lanes] bf16x8
constexpr int kPOffset = kNBuf * kSubBytes;
constexpr int kPHalf = 2 * 2 * 64 * 16;
// Metadata rings (per sub-tile, 64 copies of 32 entries): int32 ring_idx[16][64]
// (sparse slot indices) and ring_pg[8][64] (sparse: each slot's token row, or -1;
// dense: the sub-tile's page)
constexpr int kRingIdx = 16;
constexpr int kRingPg = 8;
constexpr int kMetaOffset = kPOffset + 2 * kPHalf;
constexpr int kMetaBytes = (kRingIdx + kRingPg) * 64 * 4;
constexpr int kFlagOffset = kMetaOffset + kMetaBytes;  // int32 per-wave flags[8]
constexpr int kXOffset = kFlagOffset + 64;             // float row exchange [3][64]
constexpr int kLdsBytes = kXOffset + 3 * 64 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// epilogue staging of the output tile in the tile buffers: rows padded by 16 bytes
constexpr int kOutRowBf16 = kDV * 2 + 16;
constexpr int kOutRowF32 = kDV * 4 + 16;
static_assert(kRowTile * kOutRowF32 <= kNBuf * kSubBytes, "output staging fits the tile buffers");
constexpr int kFp8Loads = 9;  // vector memory operations of one wave's FP8 load (4 codes, 4 scales, RoPE)
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;
constexpr int kAhead = 4;  // K fragments read ahead of their score MFMAs

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void tile_barrier_drain() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier after waiting for all but this wave's N most recent vector memory
// loads, through the builtin whose wait the compiler's wait-count pass sees.
template <int N>
__device__ __forceinline__ void barrier_keep_seen() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
}

// Offset past the pool for tokens no query row attends (pool-wide buffer loads
// read zeros there): the pool is at most this many bytes, and this plus a
// token's 656 bytes does not wrap.
constexpr uint32_t kPastPoolF8 = 0xFFFFF000u;

// A token of zeros: the source for tokens no query row attends when the pool
// is too large for 32-bit offsets (then each token's address is a pointer).
__device__ __attribute__((aligned(64))) uint8_t g_zero_fp8_token[kFp8TokenBytes] = {0};

// FP8 registers of one wave's share of a sub-tile: for k = 0..3 the 8 codes of
// dims 8 lane .. of token 8 k + wave and their scale (scale lane / 16), and 8
// bytes of RoPE (dims 512 + 4 (lane % 16) ..) of token 8 (lane / 16) + wave.  A
// wave thus writes 64 consecutive 16-byte chunks of one token per store
// (conflict-free LDS writes) from 512 consecutive code bytes.
struct RawFp8 {
  u32x2 v[4];
  float sc[4];
  u32x2 r;
};
struct Fp8Rows {
  int v[4];
};

template <bool SPARSE, bool BUFG>
__global__ __launch_bounds__(kThreads8, 1) void mla_decode_fp8_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  MLA_LDS char* pbuf = smem + kPOffset;
  MLA_LDS int32_t* ring_idx = (MLA_LDS int32_t*)(smem + kMetaOffset);
  MLA_LDS int32_t* ring_pg = ring_idx + kRingIdx * 64;
  MLA_LDS int32_t* wflag = (MLA_LDS int32_t*)(smem + kFlagOffset);
  MLA_LDS float* xrow = (MLA_LDS float*)(smem + kXOffset);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wave_s < 4;
  const int l16 = lane & 15, h4 = lane >> 4;  // 16x16 operand row / k-group
  const int l32 = lane & 31, h2 = lane >> 5;  // 32x32 operand row / k-group
  const int rg = (wave_s >> 1) & 1, tb = wave_s & 1;  // score waves
  const int cv = wave_s & 3;                          // PV waves

  // workgroup -> (worker, row tile), as in the general kernel
  int w, rt;
  {
    const int g = blockIdx.x;
    if (p.n_rt == 1) {
      w = g;
      rt = 0;
    } else if ((p.W & 15) == 0) {
      const int grp = g / (16 * p.n_rt), k = (g >> 3) % (2 * p.n_rt);
      rt = k >> 1;
      w = grp * 16 + 2 * (g & 7) + (k & 1);
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
  const int hi0 = ent[5], nsplit0 = ent[6];  // the first piece's end tile and its stream's splits
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int32_t* first = p.meta + meta_tile_first(p.W, p.n_streams);

  for (int stream = bs; stream <= es && stream < p.n_streams; ++stream) {
    // The first piece comes from the schedule entry alone, so its Q, metadata
    // and tile loads wait for one metadata round trip; later pieces read their
    // stream's tile count and splits.
    int lo = 0, hi, sid, nsplit;
    if (stream == bs) {
      lo = bt0;
      hi = hi0;
      sid = split0;
      nsplit = nsplit0;
    } else {
      hi = stream == es ? et : first[stream + 1] - first[stream];
      sid = split_off[stream];
      nsplit = split_off[stream + 1] - sid;
    }
    if (hi <= lo) continue;
    const bool final_out = nsplit == 1;

    const int b = SPARSE ? stream / p.s_q : stream;
    const int64_t row_base = (int64_t)stream * p.R_stream;
    const int seqlen = __builtin_amdgcn_readfirstlane(p.seqlens[b]);
    const int32_t* bt_row = p.block_table + (int64_t)b * p.max_blocks;
    const int32_t* idx_row = SPARSE ? p.indices + (int64_t)stream * p.topk : nullptr;
    const __amdgpu_buffer_rsrc_t bt_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)bt_row, 0, p.max_blocks * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t idx_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)idx_row, 0, SPARSE ? p.topk * 4 : 0, kBufferFlags);
    // sub-tiles [u0, u1): 32 tokens (dense) or 32 index slots (sparse) each
    const int limit = SPARSE ? p.topk : seqlen;
    const int u0 = 2 * lo;
    const int u1 = min(2 * hi, (limit + kSub - 1) / kSub);
    auto buffer = [&](int u) -> MLA_LDS char* { return smem + ((unsigned)(u - u0) & (kNBuf - 1)) * kSubBytes; };

    // ---- metadata ---------------------------------------------------------------
    // What a sub-tile's loads need (its page, or each slot's token row) sits in
    // LDS rings written ahead: the prologue fills them by direct loads; then
    // round u loads into VGPRs the indices of sub-tile u + 8 (sparse, wave 4) and
    // the pages of sub-tile u + 6 (wave 5; sparse: of its slots' indices), and the
    // same waves write them into the rings in round u + 1, after the store that
    // waits for the loads issued after them (a wait for a register load waits for
    // every older load).  They are PV waves: a wave issues about one VALU
    // instruction every 7 clocks, and the score waves carry more per round.
    // Sparse rings then hold each slot's token row (page * 64 + index % 64, or -1
    // when the slot is not attended).
    auto slot_ok = [&](int u) { return u < u1 && u * kSub + l32 < p.topk; };  // sparse slot l32 exists
    auto idx_slot = [&](int x) -> MLA_LDS int32_t* { return ring_idx + (x & (kRingIdx - 1)) * 64; };
    auto pg_slot = [&](int x) -> MLA_LDS int32_t* { return ring_pg + (x & (kRingPg - 1)) * 64; };
    auto fetch_idx = [&](int x) {
      const int si = min(x * kSub + l32, p.topk - 1);
      buffer_load_lds4(idx_rs, (MLA_LDS void*)idx_slot(x), (uint32_t)si * 4u);
    };
    auto fetch_pg = [&](int x) {
      const int idx = idx_slot(x)[l32];
      const bool ok = slot_ok(x) && idx >= 0;
      buffer_load_lds4(bt_rs, (MLA_LDS void*)pg_slot(x), (uint32_t)(ok ? idx >> 6 : 0) * 4u);
    };
    auto fetch_page = [&](int x) {
      buffer_load_lds4(bt_rs, (MLA_LDS void*)pg_slot(x), (uint32_t)(min(x, u1 - 1) >> 1) * 4u);
    };
    auto meta_idx_load = [&](int u) -> int {  // sparse: the indices of sub-tile u + 8
      int z = 0;
      asm volatile("" : "+v"(z));  // a per-lane index, so this is a vector load
      return idx_row[min((u + 8) * kSub + l32, p.topk - 1) + z];
    };
    // (i6: the ring's index of slot l32 of sub-tile u + 6, read by the caller)
    auto meta_pg_load = [&](int u, int i6) -> int {  // the pages of sub-tile u + 6
      int z = 0;
      asm volatile("" : "+v"(z));
      if constexpr (SPARSE) return bt_row[(slot_ok(u + 6) && i6 >= 0 ? i6 >> 6 : 0) + z];
      return bt_row[(min(u + 6, u1 - 1) >> 1) + z];
    };
    auto fp8_token_row = [&](int x, int pg) -> int {
      const int i = idx_slot(x)[l32];
      return slot_ok(x) && i >= 0 ? pg * kPage + (i & 63) : -1;
    };
    // ---- FP8 staging (every wave: tokens 8 k + wave) -------------------------------
    auto fp8_rows = [&](int u) -> Fp8Rows {
      Fp8Rows t;
#pragma unroll
      for (int k = 0; k < 4; ++k) t.v[k] = SPARSE ? pg_slot(u)[8 * k + wave_s] : (k == 0 ? pg_slot(u)[0] : 0);
      return t;
    };
    auto load_fp8 = [&](int u, RawFp8& r, const Fp8Rows& rows) {
      // per-lane offsets: kept live across the loop where registers allow (pool
      // offsets: recomputing them cost the score wave ~27 VALU instructions a
      // round, c4 -6 %), else recomputed from an opaque copy of the lane
      int lo2 = lane;
      if constexpr (!BUFG) asm volatile("" : "+v"(lo2));
      if constexpr (BUFG) {
        // One resource over the pool: a token's byte offset, or past the pool.
        // (A select between a token's pointer and the zero token made the
        // compiler reload the zero token's address by a scalar load in the
        // loop, and the wait for that load drained the wave's LDS operations,
        // twice per round: c4 -4 % without it.)
        const __amdgpu_buffer_rsrc_t pool_rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, 0, p.pool_records, kBufferFlags);
        uint32_t toff[4];
        if constexpr (SPARSE) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int tk = __builtin_amdgcn_readfirstlane(rows.v[k]);
            toff[k] = u < u1 && tk >= 0 ? (uint32_t)tk * (uint32_t)kFp8TokenBytes : kPastPoolF8;
          }
        } else {
          const int valid = u < u1 ? seqlen - u * kSub : 0;
          const int page = __builtin_amdgcn_readfirstlane(rows.v[0]);
          const uint32_t base = (uint32_t)(page * kPage + (u & 1) * kSub) * (uint32_t)kFp8TokenBytes;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int t = 8 * k + wave_s;
            toff[k] = t < valid ? base + (uint32_t)t * (uint32_t)kFp8TokenBytes : kPastPoolF8;
          }
        }
        const uint32_t ul = (uint32_t)lo2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          r.v[k] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(pool_rs, toff[k] + 8u * ul, 0, 0));
          r.sc[k] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(pool_rs, toff[k] + (uint32_t)kFp8Dims + 4u * (ul >> 4), 0, 0));
        }
        const uint32_t kr = ul >> 4;
        const uint32_t tr = kr == 0 ? toff[0] : kr == 1 ? toff[1] : kr == 2 ? toff[2] : toff[3];
        r.r = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(pool_rs, tr + (uint32_t)(kFp8Dims + 16) + 8u * (ul & 15u), 0, 0));
        return;
      }
      const uint8_t* pt[4];
      if constexpr (SPARSE) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tk = __builtin_amdgcn_readfirstlane(rows.v[k]);
          pt[k] = u < u1 && tk >= 0 ? p.kv + (int64_t)tk * kFp8TokenBytes : g_zero_fp8_token;
        }
      } else {
        // past the split the ring slot may never have been written: its page is not used
        const int valid = u < u1 ? seqlen - u * kSub : 0;  // tokens of the sub-tile in the sequence
        const int page = __builtin_amdgcn_readfirstlane(rows.v[0]);
        const uint8_t* base = p.kv + ((int64_t)page * kPage + (u & 1) * kSub) * kFp8TokenBytes;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = 8 * k + wave_s;
          pt[k] = t < valid ? base + t * kFp8TokenBytes : g_zero_fp8_token;
        }
      }
      // unsigned lane offsets: the loads take the scalar token address plus a
      // 32-bit per-lane offset
      const uint32_t ul = (uint32_t)lo2;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r.v[k] = *(const u32x2*)(pt[k] + 8u * ul);
        r.sc[k] = *(const float*)(pt[k] + (uint32_t)kFp8Dims + 4u * (ul >> 4));
      }
      // RoPE bytes: lanes 16 k .. 16 k + 15 cover token 8 k + wave
      const uint32_t kr = ul >> 4;
      const uint8_t* prr = kr == 0 ? pt[0] : kr == 1 ? pt[1] : kr == 2 ? pt[2] : pt[3];
      r.r = *(const u32x2*)(prr + (uint32_t)(kFp8Dims + 16) + 8u * (ul & 15u));
    };
    // Token 8 k + wave's swizzle is 4 bit1(wave) + 2 (k & 1), so the store
    // address of chunk `lane` is one of two per-lane bases plus 8 k token rows.
    auto store_fp8 = [&](const RawFp8& r, MLA_LDS char* buf) {
      int lo2 = lane;
      if constexpr (!BUFG) asm volatile("" : "+v"(lo2));
      const int b0 = (wave_s * kTokenChunks + (lo2 ^ (4 * ((wave_s >> 1) & 1)))) * 16;
      const int b1 = (wave_s * kTokenChunks + (lo2 ^ (4 * ((wave_s >> 1) & 1) + 2))) * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x2 a = dequant4(r.v[k].x, r.sc[k]), c = dequant4(r.v[k].y, r.sc[k]);
        *(MLA_LDS u32x4*)(buf + ((k & 1) ? b1 : b0) + 8 * k * kBf16TokenBytes) = u32x4{a.x, a.y, c.x, c.y};
      }
      const int tr = 8 * (lo2 >> 4) + wave_s;
      *(MLA_LDS u32x2*)(buf + tile_slot(tr, 64 + ((lo2 & 15) >> 1)) * 16 + 8 * (lo2 & 1)) = r.r;
    };
    // sparse: the prologue's pages become token rows (waves 0..5, one sub-tile each)
    auto rows_from_pages = [&]() {
      if constexpr (SPARSE) {
        if (wave_s < 6) {
          const int x = u0 + wave_s;
          const int tk = fp8_token_row(x, pg_slot(x)[l32]);
          pg_slot(x)[lane] = tk;
        }
        lds_barrier();
      }
    };

    if (score_wave) {
      // ================================ score waves ================================
      // Dense visibility, as in the dense kernel (causal: query token i sees
      // [0, seqlen - s_q + 1 + i)); sparse: the slots whose ring entry is a token.
      const int vis_min = p.causal ? max(seqlen - p.s_q + 1, 0) : seqlen;
      int vis_row[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        vis_row[rb] = p.causal ? min(max(seqlen - p.s_q + 1 + (rt * kRowTile + 32 * rg + 16 * rb + l16) / p.h_q, 0),
                                     seqlen)
                               : seqlen;
      int kofs[2];
      {
        const int t = 16 * tb + l16;
        const int sw = tile_swizzle(t);
#pragma unroll
        for (int m = 0; m < 2; ++m) kofs[m] = t * kBf16TokenBytes + (((4 * m + h4) ^ sw) << 4);
      }
      auto kread = [&](MLA_LDS char* kb, int kk) -> bf16x8 {
        return *(MLA_LDS bf16x8*)(kb + kofs[kk & 1] + (kk >> 1) * 128);
      };
      auto pw_off = [&](int rb) -> int {
        return ((rg * 2 + tb) * 64 + 16 * rb + l16 + 32 * (h4 >> 1)) * 16 + 8 * (h4 & 1);
      };
      auto stage_q = [&](int h, MLA_LDS char* buf) {
        const int r0 = rt * kRowTile + 32 * h;
        const int nrows = __builtin_amdgcn_readfirstlane(min(max(p.R_stream - r0, 0), 32));
        const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.q + (row_base + r0) * kDQK), 0, nrows * kBf16TokenBytes, kBufferFlags);
        int to = tid;
        asm volatile("" : "+v"(to));
#pragma unroll
        for (int k = 0; k < kSubBytes / 16 / 256; ++k) {
          const int sl = k * 256 + to;
          const int t = sl / kTokenChunks;
          buffer_load_lds16(q_rs, (MLA_LDS void*)(buf + k * 4096 + wave_s * 1024),
                            (uint32_t)(t * kBf16TokenBytes + ((sl - t * kTokenChunks) ^ tile_swizzle(t)) * 16));
        }
      };
      // attended mask of sub-tile u's 32 slots (sparse; from the token-row ring)
      auto sparse_mask = [&](int u) -> uint32_t { return (uint32_t)__ballot(pg_slot(u)[l32] >= 0); };
      auto mask_scores = [&](int u, int rb, f32x4& v, uint32_t tmask) {
        const bool full = SPARSE ? tmask == 0xFFFFFFFFu : (u + 1) * kSub <= vis_min;
        if (!full) {
          asm volatile("");  // a real branch: full sub-tiles skip the masking
          int tok0 = 16 * tb + 4 * h4;
          asm volatile("" : "+v"(tok0));
          const int vcount = vis_row[rb] - u * kSub - tok0;
          const uint32_t lmask = tmask >> tok0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = SPARSE ? ((lmask >> e) & 1u) != 0 : e < vcount;
            v[e] = ok ? v[e] : kNegInf;
          }
        }
      };
      auto row_max16 = [&](float v) -> float {
        v = fmaxf(v, __shfl_xor(v, 16));
        return fmaxf(v, __shfl_xor(v, 32));
      };

      // Reference maximum per row, fixed for the split, with a restart on
      // overflow (as in the dense kernel).
      float m_ref[2] = {kNegInf, kNegInf};
      int pass = 0;
      bool redo;
      do {
        float l_sum[2] = {0.f, 0.f}, m_seen[2] = {kNegInf, kNegInf};
        bool overflow = false;
        // ---- prologue ----------------------------------------------------------------
        // Q goes through the buffers of sub-tiles u0 + 2 and u0 + 3 before they hold
        // tiles (the PV waves fill the rings meanwhile)
        stage_q(0, buffer(u0 + 2));
        stage_q(1, buffer(u0 + 3));
        if constexpr (SPARSE) lds_barrier();
        lds_barrier();
        rows_from_pages();
        // sub-tiles u0 .. u0 + 2 loaded at once (a third register set is free
        // before Q and the accumulators are), u0 and u0 + 1 stored
        RawFp8 raw, raw1, raw2;
        load_fp8(u0, raw, fp8_rows(u0));
        load_fp8(u0 + 1, raw1, fp8_rows(u0 + 1));
        load_fp8(u0 + 2, raw2, fp8_rows(u0 + 2));
        store_fp8(raw, buffer(u0));
        store_fp8(raw1, buffer(u0 + 1));
        raw = raw2;
        // Q's direct loads are older than the 9 register loads just issued
        barrier_keep_seen<kFp8Loads>();
        bf16x8 qf[2][18];
        {
          int lo2 = lane;
          asm volatile("" : "+v"(lo2));
          MLA_LDS char* qb = buffer(u0 + 2 + rg);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int t = 16 * rb + (lo2 & 15);
            const int sw = tile_swizzle(t);
#pragma unroll
            for (int kk = 0; kk < 18; ++kk)
              qf[rb][kk] = *(MLA_LDS bf16x8*)(qb + t * kBf16TokenBytes + (((4 * (kk & 1) + (lo2 >> 4)) ^ sw) << 4) +
                                               (kk >> 1) * 128);
          }
        }
        bf16x8 kf[kAhead];
        f32x4 s[2];
        // S^T of the sub-tile in kb; `step(kk)` runs after the MFMAs of k-step kk
        auto scores = [&](MLA_LDS char* kb, bool self, auto step) __attribute__((always_inline)) {
          if (self)
#pragma unroll
            for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(kb, kk);
          s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
          s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk % kAhead], qf[rb][kk], s[rb], 0, 0, 0);
            if (kk + kAhead < 18) kf[kk % kAhead] = kread(kb, kk + kAhead);
            step(kk);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        // P = 2^(scale_log2 S - m_ref) into LDS; raw-score overflow threshold
        float thr[2], msafe[2];
        auto set_ref = [&]() {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            thr[rb] = m_ref[rb] == kNegInf ? kNegInf : (m_ref[rb] + kRefRoom) / p.scale_log2;
            msafe[rb] = m_ref[rb] == kNegInf ? 0.f : m_ref[rb];
          }
        };
        auto softmax = [&](int u, uint32_t tmask) __attribute__((always_inline)) {
          f32x4 vm[2] = {s[0], s[1]};
          if (SPARSE ? tmask != 0xFFFFFFFFu : (u + 1) * kSub > vis_min) {
            asm volatile("");  // a real branch: full sub-tiles skip the masking
            int tok0 = 16 * tb + 4 * h4;
            asm volatile("" : "+v"(tok0));
            if constexpr (SPARSE) {
              // the slots are the same for both row blocks
              const uint32_t lmask = tmask >> tok0;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool ok = ((lmask >> e) & 1u) != 0;
                vm[0][e] = ok ? vm[0][e] : kNegInf;
                vm[1][e] = ok ? vm[1][e] : kNegInf;
              }
            } else {
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) {
                const int vcount = vis_row[rb] - u * kSub - tok0;
#pragma unroll
                for (int e = 0; e < 4; ++e) vm[rb][e] = e < vcount ? vm[rb][e] : kNegInf;
              }
            }
          }
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const f32x4 v = vm[rb];
            const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
            m_seen[rb] = fmaxf(m_seen[rb], mx);
            overflow |= mx > thr[rb];
            float pe[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], p.scale_log2, -msafe[rb]));
            l_sum[rb] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
            bf16x2 p01, p23;
            p01.x = (__bf16)pe[0];
            p01.y = (__bf16)pe[1];
            p23.x = (__bf16)pe[2];
            p23.y = (__bf16)pe[3];
            *(MLA_LDS u32x2*)(pbuf + (u & 1) * kPHalf + pw_off(rb)) =
                u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
          }
        };
        const uint32_t tmask0 = SPARSE ? sparse_mask(u0) : 0u;
        scores(buffer(u0), true, [](int) {});
        if (pass == 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            f32x4 v = s[rb];
            mask_scores(u0, rb, v, tmask0);
            const float mx = row_max16(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            if (h4 == 0) xrow[tb * 64 + 32 * rg + 16 * rb + l16] = mx;
          }
        }
        lds_barrier();  // every wave has read Q; the row maxima are visible
        if (pass == 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int r = 32 * rg + 16 * rb + l16;
            const float m0 = fmaxf(xrow[r], xrow[64 + r]) * p.scale_log2;
            m_ref[rb] = m0 == kNegInf ? kNegInf : m0 + kRefLift;
          }
        }
        set_ref();
        // round u0: sub-tile u0 + 2 into Q's first buffer, sub-tile u0 + 3 into the
        // registers
        store_fp8(raw, buffer(u0 + 2));
        load_fp8(u0 + 3, raw, fp8_rows(u0 + 3));
        softmax(u0, tmask0);
        if (u0 + 1 < u1)
#pragma unroll
          for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(buffer(u0 + 1), kk);
        lds_barrier();  // end of round u0: sub-tile u0 + 2 is in LDS
        // ---- rounds ------------------------------------------------------------------
        // round u: S of sub-tile u; after its first MFMAs this wave's share of
        // sub-tile u + 2 goes to LDS and the share of sub-tile u + 3 is loaded;
        // then the softmax and the first K fragments of sub-tile u + 1.
        for (int u = u0 + 1; u < u1; ++u) {
          // the ring reads of the round first: a wait for an LDS read also waits
          // for the stores issued before it (the sparse mask's entry is tested
          // after the scores, so that its wait does not hold the first MFMAs)
          int tmv = SPARSE ? pg_slot(u)[l32] : 0;
          const Fp8Rows rows3 = fp8_rows(u + 3);
          MLA_LDS char* nxt = buffer(u + 2);
          scores(buffer(u), false, [&](int kk) __attribute__((always_inline)) {
            if (kk == 1) store_fp8(raw, nxt);
            if (kk == 3) load_fp8(u + 3, raw, rows3);
          });
          asm volatile("" : "+v"(tmv));
          const uint32_t tmask = SPARSE ? (uint32_t)__ballot(tmv >= 0) : 0u;
          softmax(u, tmask);
          if (u + 1 < u1)
#pragma unroll
            for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(buffer(u + 1), kk);
          lds_barrier();
        }
        // ---- restart vote; l and m_ref of each row for the epilogue -------------
        const bool wave_overflow = __ballot(overflow) != 0;
        if (lane == 0) wflag[wave_s] = wave_overflow ? 1 : 0;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float l = l_sum[rb];
          l += __shfl_xor(l, 16);
          l += __shfl_xor(l, 32);
          int lo2 = lane;
          asm volatile("" : "+v"(lo2));
          const int r = 32 * rg + 16 * rb + (lo2 & 15);
          if (lo2 < 16) {
            xrow[tb * 64 + r] = l;
            if (tb == 0) xrow[128 + r] = m_ref[rb];
          }
        }
        // the register loads past the last round are drained before the barrier
        tile_barrier_drain();
        redo = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) redo |= wflag[i] != 0;
        redo = redo && pass == 0;
        ++pass;
        if (redo) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float ms = row_max16(m_seen[rb]);
            if (h4 == 0) xrow[tb * 64 + 32 * rg + 16 * rb + l16] = ms;
          }
          __syncthreads();
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int r = 32 * rg + 16 * rb + l16;
            const float m0 = fmaxf(xrow[r], xrow[64 + r]) * p.scale_log2;
            m_ref[rb] = m0 == kNegInf ? kNegInf : m0 + kRefLift;
          }
        }
      } while (redo);
    } else {
      // ================================= PV waves =================================
      int vofs[2];
      {
        const int q = (lane & 15) >> 2;
        const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int tok = 8 * h2 + q;
        const int sw = tile_swizzle(tok);
        const int sb = sw >> 2;
        const int base = tok * kBf16TokenBytes + 256 * cv + ((cl ^ (sw & 3)) << 4) + 8 * (lane & 1);
        vofs[0] = base + 64 * sb;
        vofs[1] = base - 64 * sb;
      }
      auto vread = [&](MLA_LDS char* vb, int s2, int ct) -> bf16x8 {
        const int o = vofs[ct & 1] + 64 * ct + 16 * s2 * kBf16TokenBytes;
        const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + o));
        const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + o + 4 * kBf16TokenBytes));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      auto pread = [&](int par, int rb, int s2) -> bf16x8 {
        return *(MLA_LDS bf16x8*)(pbuf + par * kPHalf + ((rb * 2 + s2) * 64 + lane) * 16);
      };

      f32x16 acc[2][4];  // O^T: [row block][32-column block]
      bf16x8 va[2][4];   // V^T of the sub-tile whose PV comes next
      int pass = 0;
      bool redo;
      do {
        // ---- prologue ----------------------------------------------------------------
        // the ring entries of sub-tiles u0 .. u0 + 5 (pages) and, sparse, u0 .. u0 + 7
        // (indices), two sub-tiles per wave
        {
          const int x = cv;
          if constexpr (SPARSE) {
            fetch_idx(u0 + x);
            fetch_idx(u0 + x + 4);
            tile_barrier_drain();
            fetch_pg(u0 + x);
            if (x < 2) fetch_pg(u0 + x + 4);
          } else {
            fetch_page(u0 + x);
            if (x < 2) fetch_page(u0 + x + 4);
          }
          tile_barrier_drain();
        }
        rows_from_pages();
        // sub-tiles u0 .. u0 + 2 loaded at once (a third register set is free
        // before Q and the accumulators are), u0 and u0 + 1 stored
        RawFp8 raw, raw1, raw2;
        load_fp8(u0, raw, fp8_rows(u0));
        load_fp8(u0 + 1, raw1, fp8_rows(u0 + 1));
        load_fp8(u0 + 2, raw2, fp8_rows(u0 + 2));
        store_fp8(raw, buffer(u0));
        store_fp8(raw1, buffer(u0 + 1));
        raw = raw2;
        barrier_keep_seen<kFp8Loads>();  // sub-tiles u0 and u0 + 1 are in LDS
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) va[s2][ct] = vread(buffer(u0), s2, ct);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][ct][e] = 0.f;
        lds_barrier();  // every score wave has read Q
        // round u0: sub-tile u0 + 2 into Q's first buffer, sub-tile u0 + 3 into the
        // registers
        store_fp8(raw, buffer(u0 + 2));
        // the metadata loads and ring writes are waves 4 and 5's
        int fmi = 0, fmp = 0;
        if (SPARSE && wave_s == 4) fmi = meta_idx_load(u0);
        if (wave_s == 5) fmp = meta_pg_load(u0, SPARSE ? idx_slot(u0 + 6)[l32] : 0);
        load_fp8(u0 + 3, raw, fp8_rows(u0 + 3));
        lds_barrier();  // end of round u0
        // ---- rounds ------------------------------------------------------------------
        // round u: P of sub-tile u - 1; this wave's share of sub-tile u + 2 into LDS;
        // the share of sub-tile u + 3 into the registers; P V of sub-tile u - 1 with
        // V^T of sub-tile u read between the MFMAs
        auto round = [&](const int u, MLA_LDS char* __restrict__ kb, MLA_LDS char* __restrict__ nxt)
                         __attribute__((always_inline)) {
          // the ring entries of sub-tile u + 3 first: a wait for an LDS read also
          // waits for the stores issued before it
          const Fp8Rows rows3 = fp8_rows(u + 3);
          const int i6 = SPARSE ? idx_slot(u + 6)[l32] : 0;
          bf16x8 pp[2][2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) pp[rb][s2] = pread((u - 1) & 1, rb, s2);
          store_fp8(raw, nxt);
          // round u - 1's metadata into the rings, round u's loaded (sparse: the
          // indices by wave 4, the token rows by wave 5)
          if (SPARSE && wave_s == 4) {
            idx_slot(u + 7)[lane] = fmi;
            fmi = meta_idx_load(u);
          }
          if (wave_s == 5) {
            pg_slot(u + 5)[lane] = SPARSE ? fp8_token_row(u + 5, fmp) : fmp;
            fmp = meta_pg_load(u, i6);
          }
          load_fp8(u + 3, raw, rows3);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][ct], pp[rb][s2], acc[rb][ct], 0, 0, 0);
              va[s2][ct] = vread(kb, s2, ct);
              __builtin_amdgcn_sched_barrier(0);
            }
          lds_barrier();
        };
        for (int u = u0 + 1; u < u1; ++u) round(u, buffer(u), buffer(u + 2));
        // P V of the last sub-tile
        {
          bf16x8 pp[2][2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) pp[rb][s2] = pread((u1 - 1) & 1, rb, s2);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][ct], pp[rb][s2], acc[rb][ct], 0, 0, 0);
        }
        if (lane == 0) wflag[wave_s] = 0;
        tile_barrier_drain();
        redo = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) redo |= wflag[i] != 0;
        redo = redo && pass == 0;
        ++pass;
        if (redo) __syncthreads();  // the score waves exchange the rows' maxima
      } while (redo);

      // ---- epilogue: normalised rows into the free tile buffers -------------------
      int lo2 = lane;
      asm volatile("" : "+v"(lo2));
      const int col = 128 * cv + 4 * (lo2 >> 5);
      const int lrow = lo2 & 31;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int rho = 32 * rb + lrow;  // row within the tile
        const float lj = xrow[rho] + xrow[64 + rho];
        const float mj = xrow[128 + rho];
        const int rowj = rt * kRowTile + rho;
        const bool empty = !(lj > 0.f);
        const float inv = empty ? 0.f : 1.f / lj;
        const float lse_v = empty ? kNegInf : (mj + __log2f(lj)) * 0.69314718055994531f;
        if (final_out) {
          MLA_LDS char* orow = smem + rho * kOutRowBf16 + col * 2;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& a = acc[rb][ct];
              bf16x2 v0, v1;
              v0.x = (__bf16)(a[4 * i + 0] * inv);
              v0.y = (__bf16)(a[4 * i + 1] * inv);
              v1.x = (__bf16)(a[4 * i + 2] * inv);
              v1.y = (__bf16)(a[4 * i + 3] * inv);
              *(MLA_LDS u32x2*)(orow + (ct * 32 + 8 * i) * 2) =
                  u32x2{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1)};
            }
          if (cv == 0 && lo2 < 32 && rowj < p.R_stream) p.lse[row_base + rowj] = lse_v;
        } else {
          MLA_LDS char* prow = smem + rho * kOutRowF32 + col * 4;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& a = acc[rb][ct];
              *(MLA_LDS f32x4*)(prow + (ct * 32 + 8 * i) * 4) =
                  f32x4{a[4 * i] * inv, a[4 * i + 1] * inv, a[4 * i + 2] * inv, a[4 * i + 3] * inv};
            }
          if (cv == 0 && lo2 < 32 && rowj < p.R_stream) {
            float* lp = p.part_lse + (int64_t)sid * p.R_stream + rowj;
            if (p.merge)
              store_coherent_f32(lp, lse_v);
            else
              *lp = lse_v;
          }
        }
      }
    }
    lds_barrier();
    {
      // 16-byte chunk c of the tile: row c / (chunks per row); each wave stores 1 KB runs
      const int nrows = min(p.R_stream - rt * kRowTile, kRowTile);  // rows of this tile that exist
      int to = tid;
      asm volatile("" : "+v"(to));
      if (final_out) {
        char* dst = (char*)(p.o + (row_base + rt * kRowTile) * kDV);
#pragma unroll
        for (int k = 0; k < kRowTile * kDV * 2 / 16 / kThreads8; ++k) {
          const int c = k * kThreads8 + to;
          const int row = c >> 6, off = (c & 63) * 16;
          if (row < nrows) *(u32x4*)(dst + row * (kDV * 2) + off) = *(MLA_LDS u32x4*)(smem + row * kOutRowBf16 + off);
        }
      } else {
        // a row that attends nothing in this split (lse = -inf) leaves its
        // partial output unwritten: the merge gives such a split weight 0 and
        // does not use its output
        const float lrow = xrow[to & 63] + xrow[64 + (to & 63)];
        const uint64_t live = __ballot(lrow > 0.f);
        if (p.merge) {
          merge_split_tile<kThreads8>(p, smem, kOutRowF32, stream, rt, sid, split_off[stream], nsplit, nrows, live,
                                      wflag, to);
        } else {
          char* dst = (char*)(p.part_o + ((int64_t)sid * p.R_stream + rt * kRowTile) * kDV);
#pragma unroll
          for (int k = 0; k < kRowTile * kDV * 4 / 16 / kThreads8; ++k) {
            const int c = k * kThreads8 + to;
            const int row = c >> 7, off = (c & 127) * 16;
            if (row < nrows && ((live >> row) & 1u)) *(u32x4*)(dst + row * (kDV * 4) + off) = *(MLA_LDS u32x4*)(smem + row * kOutRowF32 + off);
          }
        }
      }
    }
    // the next piece reuses LDS; after the last one there is nothing to wait for
    if (stream < es && stream + 1 < p.n_streams) __syncthreads();
  }
  if (p.merge && p.topk == 0) zero_empty_streams<kThreads8>(p, tid);
}

template <bool SPARSE, bool BUFG>
hipError_t launch_fp8(const DecodeParams& p, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  auto kern = mla_decode_fp8_kernel<SPARSE, BUFG>;
  const hipError_t e = set_lds_limit((const void*)kern, kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.W * p.n_rt), dim3(kThreads8), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream) {
  // pool-wide buffer loads while every token offset and the past-pool offset fit 32 bits
  const bool bufg = p.pool_records != 0 && p.pool_records <= kPastPoolF8;
  if (p.topk > 0) return bufg ? launch_fp8<true, true>(p, stream) : launch_fp8<true, false>(p, stream);
  return bufg ? launch_fp8<false, true>(p, stream) : launch_fp8<false, false>(p, stream);
}

}  // namespace mla
