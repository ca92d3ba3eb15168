// Split-KV decode kernel for the dense BF16 cache, with specialised waves
// (gfx950).
//
// What it computes is what the general decode kernel computes for a dense BF16
// cache: for each query row, softmax(scale * q K^T) V over the tokens the row
// attends, a token's 576-dim latent being K and its first 512 dims V (FlashMLA
// source walk-through, data-loading section), and the natural log-sum-exp of
// the scaled scores; a stream handled by one worker gets its final o and lse,
// otherwise each split leaves a normalised partial o and its lse for the
// combine kernel (same page, scheduling and combine sections).
//
// Mapping.  One workgroup of 8 waves owns 64 query rows of one stream and walks
// its tile range in 32-token sub-tiles.  Waves w and w + 4 run on the same SIMD,
// and the two of a SIMD take different roles, so that one wave's LDS and
// barrier waits are covered by the other's MFMAs (the pages' warpgroup
// ping-pong, here between the two waves of a SIMD):
//  - score waves 0..3: wave w computes S^T for rows 32 rg .. 32 rg + 31
//    (rg = w / 2) and tokens 16 tb .. 16 tb + 15 (tb = w % 2) of each sub-tile
//    over all 576 dims on v_mfma_f32_16x16x32_bf16, its 32 Q rows in VGPRs, so
//    each K fragment read from LDS feeds two MFMAs (with 16 rows per wave every
//    K byte was read by four waves, and the K reads were most of the LDS
//    traffic); then the softmax against a per-row reference fixed for the split,
//    and the bf16 P block into LDS;
//  - PV waves 4..7: wave 4 + c owns O columns 128 c .. 128 c + 127 for all 64
//    rows (O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, V^T through
//    ds_read_b64_tr_b16), and issues every direct global->LDS load of the tiles
//    and of the page ring.
// Round u (one workgroup barrier each): the score waves compute S and P of
// sub-tile u; the PV waves issue the loads of sub-tile u + 3 (into the buffer
// that sub-tile u - 1 has left), multiply P V of sub-tile u - 1, and read V^T of
// sub-tile u for the next round.  Sub-tile u is read in round u only, so of
// the four 36 KB tile buffers one is read and three are landing.
#include "mla_device.hpp"

namespace mla {
namespace {

constexpr int kThreads8 = 512;  // 8 waves
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRefLift = 32.0f;  // log2 units
constexpr float kRefRoom = 88.0f;
constexpr int kSub = 32;                           // tokens per sub-tile
constexpr int kSubBytes = kSub * kBf16TokenBytes;  // 36864
constexpr int kNBuf = 4;
// P exchange: [2 (sub-tile parity)][2 row blocks of 32][2 k-steps of 16 tokens][64 lanes] bf16x8
constexpr int kPOffset = kNBuf * kSubBytes;
constexpr int kPHalf = 2 * 2 * 64 * 16;
// page ring: the cache page of each of 8 sub-tiles (64 copies)
constexpr int kRing = 8;
constexpr int kRingOffset = kPOffset + 2 * kPHalf;
constexpr int kFlagOffset = kRingOffset + kRing * 64 * 4;  // int32 per-wave flags[8]
constexpr int kXOffset = kFlagOffset + 64;                 // float row exchange [3][64]
constexpr int kLdsBytes = kXOffset + 3 * 64 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// staging: 2304 16-byte slots per sub-tile; PV-wave thread t (0..255) fills
// slots 256 k + t, k < 9
constexpr int kSlots = kSubBytes / 16;
constexpr int kLoads = kSlots / 256;
static_assert(kLoads * 256 == kSlots, "staging split");
// vector memory operations of a PV-wave thread per round: the tile pieces and
// one page-ring load
constexpr int kRoundOps = kLoads + 1;
// the page ring runs this many sub-tiles ahead of the round that fetches it
constexpr int kPageAhead = 7;
// epilogue staging of the output tile in the tile buffers: rows padded by 16 bytes
constexpr int kOutRowBf16 = kDV * 2 + 16;
constexpr int kOutRowF32 = kDV * 4 + 16;
static_assert(kRowTile * kOutRowF32 <= kNBuf * kSubBytes, "output staging fits the tile buffers");
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;
constexpr int kAhead = 4;  // K fragments read ahead of their score MFMAs

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void barrier_keep() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads8, 1) void mla_decode_dense_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  MLA_LDS char* pbuf = smem + kPOffset;
  MLA_LDS int32_t* ring = (MLA_LDS int32_t*)(smem + kRingOffset);
  MLA_LDS int32_t* wflag = (MLA_LDS int32_t*)(smem + kFlagOffset);
  MLA_LDS float* xrow = (MLA_LDS float*)(smem + kXOffset);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wave_s < 4;
  const int l16 = lane & 15, h4 = lane >> 4;  // 16x16 operand row / k-group
  const int h2 = lane >> 5;                   // 32x32 operand k-group
  const int rg = (wave_s >> 1) & 1, tb = wave_s & 1;  // score waves
  const int cv = wave_s & 3;                          // PV waves

  // workgroup -> (worker, row tile), as in the general kernel: the row tiles of
  // one worker share an XCD (XCD = blockIdx mod 8), so the second row tile reads
  // its pages from L2
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
    const int64_t row_base = (int64_t)stream * p.R_stream;
    const int seqlen = __builtin_amdgcn_readfirstlane(p.seqlens[stream]);
    const int32_t* bt_row = p.block_table + (int64_t)stream * p.max_blocks;
    const __amdgpu_buffer_rsrc_t bt_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)bt_row, 0, p.max_blocks * 4, kBufferFlags);
    // sub-tiles [u0, u1) of 32 tokens
    const int u0 = 2 * lo;
    const int u1 = min(2 * hi, (seqlen + kSub - 1) / kSub);
    auto buffer = [&](int u) -> MLA_LDS char* { return smem + ((unsigned)(u - u0) & (kNBuf - 1)) * kSubBytes; };
    auto pg_slot = [&](int x) -> MLA_LDS int32_t* { return ring + (x & (kRing - 1)) * 64; };

    if (score_wave) {
      // ================================ score waves ================================
      // Dense visibility: the tokens [0, vis) a row attends.  Non-causal: the whole
      // sequence.  Causal: the s_q query tokens are the last s_q positions, so the
      // row of query token i = row / h_q sees [0, seqlen - s_q + 1 + i) (usage
      // example of the geoz.com.cn page: causal=True).  vis_min: the smallest
      // window of the stream.
      const int vis_min = p.causal ? max(seqlen - p.s_q + 1, 0) : seqlen;
      int vis_row[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        vis_row[rb] = p.causal ? min(max(seqlen - p.s_q + 1 + (rt * kRowTile + 32 * rg + 16 * rb + l16) / p.h_q, 0),
                                     seqlen)
                               : seqlen;
      // K operand of k-step kk: token 16 tb + l16, chunk 4 kk + h4, at
      // kofs[kk & 1] + 128 (kk >> 1) (the swizzle touches the low 3 chunk bits only)
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
      // P block of row block rb of this lane (row 32 rg + 16 rb + l16, tokens
      // 16 tb + 4 h4 + e) in the layout the PV waves read: [row block rg][k-step tb]
      // [lane 16 rb + l16 + 32 (h4 / 2)] bf16x8, half h4 & 1
      auto pw_off = [&](int rb) -> int {
        return ((rg * 2 + tb) * 64 + 16 * rb + l16 + 32 * (h4 >> 1)) * 16 + 8 * (h4 & 1);
      };
      // Q rows 32 h .. 32 h + 31 of the tile into a tile buffer, in the tile layout
      // (rows in place of tokens): one copy per workgroup in 1 KB runs; rows past
      // the stream load zeros (the resource covers only existing rows)
      auto stage_q = [&](int h, MLA_LDS char* buf) {
        const int r0 = rt * kRowTile + 32 * h;
        const int nrows = __builtin_amdgcn_readfirstlane(min(max(p.R_stream - r0, 0), 32));
        const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.q + (row_base + r0) * kDQK), 0, nrows * kBf16TokenBytes, kBufferFlags);
        int to = tid;
        asm volatile("" : "+v"(to));
#pragma unroll
        for (int k = 0; k < kSlots / 256; ++k) {
          const int sl = k * 256 + to;
          const int t = sl / kTokenChunks;
          buffer_load_lds16(q_rs, (MLA_LDS void*)(buf + k * 4096 + wave_s * 1024),
                            (uint32_t)(t * kBf16TokenBytes + ((sl - t * kTokenChunks) ^ tile_swizzle(t)) * 16));
        }
      };
      auto mask_scores = [&](int u, int rb, f32x4& v) {
        if ((u + 1) * kSub > vis_min) {
          asm volatile("");  // a real branch: full sub-tiles skip the masking
          int tok0 = 16 * tb + 4 * h4;
          asm volatile("" : "+v"(tok0));
          const int vcount = vis_row[rb] - u * kSub - tok0;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = e < vcount ? v[e] : kNegInf;
        }
      };
      auto row_max16 = [&](float v) -> float {
        v = fmaxf(v, __shfl_xor(v, 16));
        return fmaxf(v, __shfl_xor(v, 32));
      };

      // Reference maximum m_ref (log2 domain, per row): the row's maximum over
      // the split's first sub-tile + kRefLift, fixed for the whole split, so
      // P = 2^(x - m_ref) stays within [2^-126, 2^(kRefLift + kRefRoom)] for every
      // score within (kRefRoom, 126 - kRefLift) of that maximum and O changes only
      // through MFMAs.  A score more than kRefRoom above m_ref, or a finite score
      // in a row whose first sub-tile was fully masked, marks the pass as
      // overflowed, and the split is recomputed with the split's true row
      // maximum as the reference (at most two passes).
      float m_ref[2] = {kNegInf, kNegInf};
      int pass = 0;
      bool redo;
      do {
        float l_sum[2] = {0.f, 0.f}, m_seen[2] = {kNegInf, kNegInf};
        bool overflow = false;
        // ---- prologue (the PV waves fetch the page ring and the first tiles) ----
        // Q goes through the buffers of sub-tiles u0 + 2 and u0 + 3 before they hold tiles
        stage_q(0, buffer(u0 + 2));
        stage_q(1, buffer(u0 + 3));
        lds_barrier();     // the ring entries have landed (PV waves)
        barrier_keep<0>();  // Q and sub-tile u0 have landed
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
        // S^T of sub-tile u (both row blocks); the first kAhead K fragments are
        // in kf unless `self`
        auto scores = [&](MLA_LDS char* kb, bool self) __attribute__((always_inline)) {
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
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        // P = 2^(scale_log2 S - m_ref) of sub-tile u into LDS.  The overflow test
        // compares the raw scores with (m_ref + kRefRoom) / scale_log2 (scale > 0),
        // which is -inf when the row has no reference yet, so that any finite
        // score then marks the pass; m_seen is kept in raw units.
        float thr[2], msafe[2];
        auto set_ref = [&]() {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            thr[rb] = m_ref[rb] == kNegInf ? kNegInf : (m_ref[rb] + kRefRoom) / p.scale_log2;
            msafe[rb] = m_ref[rb] == kNegInf ? 0.f : m_ref[rb];
          }
        };
        auto softmax = [&](int u) __attribute__((always_inline)) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            f32x4 v = s[rb];
            mask_scores(u, rb, v);
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
        scores(buffer(u0), true);
        if (pass == 0) {
          // the reference of each row from sub-tile u0 (both token-block waves of the row)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            f32x4 v = s[rb];
            mask_scores(u0, rb, v);
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
        softmax(u0);
        lds_barrier();  // end of round u0
        // ---- rounds --------------------------------------------------------------
        for (int u = u0 + 1; u < u1; ++u) {
          scores(buffer(u), u == u0 + 1);
          softmax(u);
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
        __syncthreads();
        redo = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) redo |= wflag[i] != 0;
        redo = redo && pass == 0;
        ++pass;
        if (redo) {
          // the split's row maximum over the two token-block waves of each row
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
      const int x = cv;
      // direct loads of a sub-tile: a resource over the sub-tile's tokens inside
      // the sequence (pieces past its end load zeros), from its ring entry
      // (pgv: the sub-tile's ring entry, read by the caller)
      __amdgpu_buffer_rsrc_t st_rs;
      auto stage_begin_pg = [&](int u, int pgv) {
        const int page = __builtin_amdgcn_readfirstlane(pgv);
        const uint8_t* base = p.kv + ((int64_t)page * kPage + (u & 1) * kSub) * kBf16TokenBytes;
        const int valid = __builtin_amdgcn_readfirstlane(min(max(seqlen - u * kSub, 0), kSub));
        st_rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, valid * kBf16TokenBytes, kBufferFlags);
      };
      auto stage_begin = [&](int u) { stage_begin_pg(u, pg_slot(u)[0]); };
      // source offset of this thread's piece k within the sub-tile: slot
      // 256 k + (tid - 256) holds token slot / 72, stored chunk slot % 72 (the
      // source chunk is that XOR the token's swizzle)
      uint32_t soff[kLoads];
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        const int sl = k * 256 + tid - 256;
        const int t = sl / kTokenChunks;
        soff[k] = (uint32_t)(t * kBf16TokenBytes + ((sl - t * kTokenChunks) ^ tile_swizzle(t)) * 16);
      }
      auto stage_load = [&](int k, MLA_LDS char* buf) {
        buffer_load_lds16(st_rs, (MLA_LDS void*)(buf + k * 4096 + x * 1024), soff[k]);
      };
      auto stage_all = [&](int u, MLA_LDS char* buf) {
        stage_begin(u);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) stage_load(k, buf);
      };
      // the page of sub-tile x (past the split: the split's last page, whose
      // loads stay in bounds and are not read)
      auto fetch_page = [&](int xs) {
        buffer_load_lds4(bt_rs, (MLA_LDS void*)pg_slot(xs), (uint32_t)(min(xs, u1 - 1) >> 1) * 4u);
      };
      // V^T operand (transposed reads) of k-step s2 and 32-column block ct
      // (columns 128 cv + 32 ct ..): the 4 lanes of a quad supply tokens
      // 16 s2 + 8 h2 + 4 e4 + q and each lane receives its column at those
      // tokens.  Their swizzle depends on bits 1 and 3 only (q and h2), so s2 and
      // e4 add constants; ct's low bit meets the swizzle's bit 2 (vofs[ct & 1]).
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
        // ---- prologue --------------------------------------------------------------
        fetch_page(u0 + x);
        if (x < kPageAhead - 4) fetch_page(u0 + x + 4);
        barrier_keep<0>();  // the ring entries of u0 .. u0 + 6 are visible
        // Sub-tile u0 + 1 (and later u0 + 2) is loaded even when the split ends
        // first (the resource keeps such loads in bounds; the buffer is not read),
        // so that every path issues the same loads.
        stage_all(u0, buffer(u0));
        stage_all(u0 + 1, buffer(u0 + 1));
        barrier_keep<kLoads>();  // Q and sub-tile u0 have landed
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
        // round u0: sub-tile u0 + 2 into Q's first buffer, u0 + 3 into its second
        stage_all(u0 + 2, buffer(u0 + 2));
        const bool issue0 = u0 + 3 < u1;
        if (issue0) {
          stage_all(u0 + 3, buffer(u0 + 3));
          fetch_page(u0 + kPageAhead);
        }
        if (u0 + 4 < u1) stage_begin(u0 + 4);
        // end of round u0: sub-tile u0 + 2 has landed (the score waves read its
        // first K fragments at the end of round u0 + 1)
        if (issue0)
          barrier_keep<kRoundOps>();
        else
          barrier_keep<0>();
        // ---- rounds --------------------------------------------------------------
        // round u: first the loads of sub-tile u + 3 (resource from the previous
        // round).  The compute unit's address path accepts a load instruction at
        // the rate it moves 1 KB, so the four PV waves spend about as long issuing
        // them as the score waves of the same SIMDs spend on their MFMAs.  Then
        // P V of sub-tile u - 1 with V^T of sub-tile u read between the MFMAs (the
        // softmax of the score waves runs meanwhile), then the resource of
        // sub-tile u + 4, whose ring entry is read before the MFMAs (after them it
        // cost 3 % on the compute-bound s_q = 2 workload).  (Issuing the P and ring
        // reads before the loads measured 10 % slower there.)
        auto round = [&](const int u, MLA_LDS char* __restrict__ kb, MLA_LDS char* __restrict__ nxt)
                         __attribute__((always_inline)) {
          const bool issue = u + 3 < u1;  // workgroup-uniform
          if (issue) {
#pragma unroll
            for (int k = 0; k < kLoads; ++k) stage_load(k, nxt);
            fetch_page(u + kPageAhead);
          }
          bf16x8 pp[2][2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) pp[rb][s2] = pread((u - 1) & 1, rb, s2);
          // the ring entry of sub-tile u + 4 (landed two rounds ago), read here so
          // that its latency passes under the MFMAs rather than before the barrier
          const int pg4 = pg_slot(u + 4)[0];
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
          if (u + 4 < u1) stage_begin_pg(u + 4, pg4);
          if (issue)
            barrier_keep<kRoundOps>();  // sub-tile u + 2 has landed
          else
            barrier_keep<0>();
        };
        for (int u = u0 + 1; u < u1; ++u) round(u, buffer(u), buffer(u + 3));
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
        __syncthreads();
        redo = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) redo |= wflag[i] != 0;
        redo = redo && pass == 0;
        ++pass;
        if (redo) __syncthreads();  // the score waves exchange the rows' maxima
      } while (redo);

      // ---- epilogue: normalised rows into the free tile buffers -------------------
      // (rows padded by 16 bytes against bank conflicts) so that the global
      // stores are whole contiguous runs: each lane's accumulators hold 4 columns
      // of 32 different rows
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

}  // namespace

hipError_t launch_decode_dense(const DecodeParams& p, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)mla_decode_dense_kernel, kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_decode_dense_kernel, dim3(p.W * p.n_rt), dim3(kThreads8), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace mla
