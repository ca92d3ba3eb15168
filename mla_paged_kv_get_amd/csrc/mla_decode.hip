// Split-KV decode kernel for MLA over a paged latent cache (gfx950): the sparse
// BF16 cache (index lists over a BF16 cache, also the sparse prefill).  The dense
// BF16 cache and the FP8 caches have kernels of their own with specialised waves
// (mla_decode_dense.hip, mla_decode_fp8.hip).
//
// What it computes: for each query row, softmax(scale * q K^T) V over the
// attended tokens of its stream (slot i of a query token's index list names
// cache position indices[i], -1 = not attended), where a token's 576-dim latent
// is K and its first 512 dims are V (FlashMLA source walk-through, data-loading
// section), and the natural log-sum-exp of the scaled scores.  Each worker processes the KV
// tile range the scheduler gave it; a stream handled by one worker gets its
// final o and lse here, otherwise each split leaves a normalised partial o and
// its lse for the combine kernel (same page, scheduling and combine sections).
//
// Mapping to the hardware.  One workgroup of 8 waves (two per SIMD) owns 64
// query rows of one stream; the chip runs one such workgroup per compute unit.
// Two waves per SIMD matter here: a wave's LDS reads and writes are issued at a
// fixed per-wave rate, so the second wave doubles the LDS traffic a SIMD can
// sustain, and each wave's waits (LDS, barrier) are covered by the other's MFMAs.
// Per 32-token sub-tile of the KV stream:
//   1. the sub-tile's bf16 rows are gathered into a swizzled LDS tile by direct
//      global->LDS 16-byte loads, three sub-tiles ahead; four buffers hold the
//      sub-tile being multiplied by V, the next one (whose scores are being
//      computed) and the two behind it;
//   2. scores: wave w computes S^T for 16 query rows (16 (w & 3) ..) and 16 tokens
//      (16 (w >> 2) ..) over all 576 dims on v_mfma_f32_16x16x32_bf16, with its Q
//      rows in VGPRs, so no wave needs another's partial scores;
//   3. softmax in the log2 domain against a per-row reference fixed at the start
//      of the split (see the main loop), so O and l need no rescaling; each wave
//      writes its 16 x 16 bf16 P block to LDS;
//   4. O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: wave w owns O columns
//      64 w .. 64 w + 63 for all 64 rows, reading P of the whole sub-tile from LDS
//      and V^T from the token-major tile through ds_read_b64_tr_b16.
// The steps are pipelined one sub-tile apart: round u computes the softmax of
// sub-tile u, then O += P V of sub-tile u - 1 (whose P every wave wrote in the
// previous round), then the scores of sub-tile u + 1, while sub-tile u + 2
// streams in; one workgroup barrier per round publishes all of it.
// Slots that no row attends (-1 indices, slots past the list) are loaded as
// zeros, so every wave issues the same loads per sub-tile, and their scores are
// masked to -inf.
#include "mla_device.hpp"

namespace mla {

// A token of zeros: the source for slots no query row attends.
__device__ __attribute__((aligned(64))) uint8_t g_zero_token[kBf16TokenBytes] = {0};

namespace {

constexpr int kDecThreads = 512;  // 8 waves

// Workgroup barrier that orders LDS traffic only.  __syncthreads() implies a
// release fence that also waits for every outstanding global->LDS load; this one
// leaves them in flight.  The memory clobber keeps the compiler from moving
// memory accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Also wait for every global->LDS load of this wave.
__device__ __forceinline__ void tile_barrier_drain() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct buffer loads into LDS: lane i writes 16 (or 4) bytes at dst + 16 i (4 i);
// an offset past the resource's size loads zeros.  (Kept out of lambdas: there
// the builtin makes the host pass drop the kernel.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void global_load_lds16(const void* src, MLA_LDS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rs, MLA_LDS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
}
// Workgroup barrier after waiting for this wave's LDS operations and for all but
// its N most recently issued vector memory loads (loads complete in issue order).
template <int N>
__device__ __forceinline__ void barrier_keep() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same through the builtin, whose wait the compiler's wait-count pass sees:
// afterwards it knows the older loads (direct loads into LDS included) are
// done and adds no waits of its own for them.  gfx9 s_waitcnt immediate:
// vmcnt in bits 3:0 and 15:14, expcnt in 6:4 (7: no wait), lgkmcnt in 11:8.
template <int N>
__device__ __forceinline__ void barrier_keep_seen() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int V>
struct Tag {
  static constexpr int value = V;
};

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRefLift = 32.0f;   // log2 units
constexpr float kRefRoom = 88.0f;
constexpr int kSub = 32;                               // tokens per sub-tile
constexpr int kSubBytes = kSub * kBf16TokenBytes;      // 36864
constexpr int kNBuf = 4;
// P exchange: [2 (sub-tile parity)][2 row blocks][2 k-steps][64 lanes] bf16x8
constexpr int kPOffset = kNBuf * kSubBytes;
constexpr int kPHalf = 2 * 2 * 64 * 16;
// Metadata rings (per sub-tile): int32 ring_idx[16][64] (sparse slot indices)
// and ring_pg[8][64] (their pages).
constexpr int kRingIdx = 16;
constexpr int kRingPg = 8;
constexpr int kMetaOffset = kPOffset + 2 * kPHalf;
constexpr int kMetaBytes = (kRingIdx + kRingPg) * 64 * 4;
constexpr int kFlagOffset = kMetaOffset + kMetaBytes;  // int32 per-wave flags[8]
constexpr int kXOffset = kFlagOffset + 64;             // float row exchange [3][64]
constexpr int kLdsBytes = kXOffset + 3 * 64 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// BF16 staging: 2304 16-byte slots per sub-tile; thread tid fills slots
// 512 k + tid (k < 4) and, for tid < 256, 2048 + tid.
constexpr int kSlots = kSubBytes / 16;
constexpr int kLoads = 5;
// epilogue staging of the output tile in the tile buffers: row strides of the
// bf16 output and the fp32 partial output, padded by 16 bytes
constexpr int kOutRowBf16 = kDV * 2 + 16;
constexpr int kOutRowF32 = kDV * 4 + 16;
static_assert(kRowTile * kOutRowF32 <= kNBuf * kSubBytes, "output staging fits the tile buffers");
// a gather offset past every pool the MUBUF gathers are used for (their
// resource covers at most kPastPool bytes, and kPastPool + 16 does not wrap)
constexpr uint32_t kPastPool = 0xFFFFFF00u;
static_assert(kSlots == 4 * kDecThreads + kDecThreads / 2, "staging split");
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// BUFG: token gathers as MUBUF loads against one resource over the whole KV pool
// (pools below 4 GiB), where a skipped slot's offset lies past the pool and
// loads zeros; else FLAT loads from per-lane addresses.
template <bool BUFG>
__global__ __launch_bounds__(kDecThreads, 1) void mla_decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  MLA_LDS char* pbuf = smem + kPOffset;
  MLA_LDS int32_t* ring_idx = (MLA_LDS int32_t*)(smem + kMetaOffset);
  MLA_LDS int32_t* ring_pg = ring_idx + kRingIdx * 64;
  MLA_LDS int32_t* wflag = (MLA_LDS int32_t*)(smem + kFlagOffset);
  MLA_LDS float* xrow = (MLA_LDS float*)(smem + kXOffset);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // the same, as a scalar
  const int l16 = lane & 15, h4 = lane >> 4;  // 16x16 operand row / k-group
  const int l32 = lane & 31, h2 = lane >> 5;  // 32x32 operand row / k-group
  // scores: rows 16 r4 .., tokens 16 tb .. of each sub-tile
  const int r4 = wave_s & 3, tb = wave_s >> 2;  // scalars
  const int qrow = 16 * r4 + l16;  // this lane's query row (0..63) in the score and softmax steps

  // workgroup -> (worker, row tile).  Workgroups are dealt to the 8 XCDs in turn
  // (XCD = blockIdx mod 8).  The row tiles of one worker share an XCD, so the
  // second row tile reads its pages from L2; with several row tiles and whole
  // groups of 16 workers, workers 2 x and 2 x + 1 (usually two splits of one
  // stream, which read the same Q rows) share one as well (c4: -1.3 us; with a
  // single row tile the pairing measured 3 us slower on c5 and is not used).
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

  // ---- per-lane constants -------------------------------------------------------
  // K operand of k-step kk (dims 32 kk ..): token 16 tb + l16, chunk 4 kk + h4,
  // i.e. kofs[kk & 1] + 128 (kk >> 1) (the swizzle only touches the low 3 bits).
  int kofs[2];
  {
    const int t = 16 * tb + l16;
    const int sw = tile_swizzle(t);
#pragma unroll
    for (int m = 0; m < 2; ++m) kofs[m] = t * kBf16TokenBytes + (((4 * m + h4) ^ sw) << 4);
  }
  // V^T operand (transposed reads) of k-step s2, half e4 and the parity of the
  // 32-column block: the 4 lanes of a quad supply tokens 16 s2 + 8 h2 + 4 e4 + q,
  // and each lane receives its column at those 4 tokens; columns 64 wave ..
  // The swizzle of those tokens depends on bits 1 and 3 only (q and h2), so
  // s2 and e4 add the constant 1152 (16 s2 + 4 e4): vofs holds s2 = e4 = 0.
  int vofs[2];
  {
    const int q = (lane & 15) >> 2;
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tok = 8 * h2 + q;
    const int sw = tile_swizzle(tok);
    const int sb = sw >> 2;
    const int base = tok * kBf16TokenBytes + 128 * wave_s + ((cl ^ (sw & 3)) << 4) + 8 * (lane & 1);
    vofs[0] = base + 64 * sb;
    vofs[1] = base - 64 * sb;
  }
  // P block of this lane (row qrow, tokens 16 tb + 4 h4 + e) in the layout the
  // PV step reads: [row block qrow / 32][k-step tb][lane 16 (r4 & 1) + l16 + 32 (h4 / 2)]
  // bf16x8, half h4 & 1.
  const int pw_off = (((r4 >> 1) * 2 + tb) * 64 + 16 * (r4 & 1) + l16 + 32 * (h4 >> 1)) * 16 + 8 * (h4 & 1);

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

    const int b = stream / p.s_q;  // a stream is one query token of a request
    const int64_t row_base = (int64_t)stream * p.R_stream;
    const int32_t* bt_row = p.block_table + (int64_t)b * p.max_blocks;
    const int32_t* idx_row = p.indices + (int64_t)stream * p.topk;
    // Buffer resources for the direct loads into LDS: MUBUF loads keep the
    // compiler's wait counts exact (a FLAT load into LDS makes it drain every
    // counter at each wait), and an offset past the range loads zeros.
    const __amdgpu_buffer_rsrc_t bt_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)bt_row, 0, p.max_blocks * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t idx_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)idx_row, 0, p.topk * 4, kBufferFlags);
    // sub-tiles [u0, u1) of 32 index slots
    const int u0 = 2 * lo;
    const int u1 = min(2 * hi, (p.topk + kSub - 1) / kSub);

    // Q fragments (B operand of the score MFMA): row qrow, dims 32 kk + 8 h4 ..
    // The row tile's 64 Q rows (contiguous, 1152 B each) are brought into two
    // tile buffers by direct loads in the tile layout (rows in place of tokens,
    // the same swizzle): one copy per workgroup in whole 1 KB runs, where
    // per-lane register loads would fetch every row twice (both token-block
    // waves of a row block) in 64-byte pieces.  Each wave then reads its 16 rows
    // the way it reads K.  Rows past the stream's last load as zeros: the
    // resource covers only existing rows.
    bf16x8 qf[18];
    auto buffer = [&](int u) -> MLA_LDS char* { return smem + ((unsigned)(u - u0) & (kNBuf - 1)) * kSubBytes; };
    // Waves 0..3 alone load Q (9 pieces per thread and half), so that waves 4..7
    // can fetch the ring metadata meanwhile and wait for it without waiting
    // for Q (a wave's wait for a load is a wait for all its older loads).
    auto stage_q = [&](int h, MLA_LDS char* buf) {  // rows 32 h .. 32 h + 31 of the tile; waves 0..3
      const int r0 = rt * kRowTile + 32 * h;
      const int nrows = __builtin_amdgcn_readfirstlane(min(max(p.R_stream - r0, 0), 32));
      const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.q + (row_base + r0) * kDQK), 0, nrows * kBf16TokenBytes, kBufferFlags);
      int to = tid;
      asm volatile("" : "+v"(to));  // slot offsets computed here, not kept live across the loop
#pragma unroll
      for (int k = 0; k < kSlots / (kDecThreads / 2); ++k) {
        const int sl = k * (kDecThreads / 2) + to;
        const int t = sl / kTokenChunks;
        buffer_load_lds16(q_rs, (MLA_LDS void*)(buf + k * (kDecThreads / 2 * 16) + wave_s * 1024),
                          (uint32_t)(t * kBf16TokenBytes + ((sl - t * kTokenChunks) ^ tile_swizzle(t)) * 16));
      }
    };
    auto read_q = [&](MLA_LDS char* b0, MLA_LDS char* b1) {  // rows 0..31 in b0, 32..63 in b1
      int lo = lane;
      asm volatile("" : "+v"(lo));  // recomputed here, not kept live across the loop
      const int t = 16 * (r4 & 1) + (lo & 15);
      const int sw = tile_swizzle(t);
      MLA_LDS char* qb = (r4 >> 1) ? b1 : b0;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk)
        qf[kk] = *(MLA_LDS bf16x8*)(qb + t * kBf16TokenBytes + (((4 * (kk & 1) + (lo >> 4)) ^ sw) << 4) +
                                    (kk >> 1) * 128);
    };

    // O^T accumulators: [row block][32-column block], columns 64 wave + 32 ct ..
    f32x16 acc[2][2];

    // ---- per sub-tile metadata ----------------------------------------------------
    // Round u issues the direct global->LDS loads of sub-tile u + 3, waited for at
    // the end of the next round.  What a round needs to know about a sub-tile (the
    // index and page of each of its 32 slots) was fetched earlier by direct loads
    // into LDS rings (16 sub-tiles of indices, 8 of pages): round u fetches the
    // indices of sub-tile u + 8 and the pages of sub-tile u + 6's indices; such a
    // load has landed and is visible two rounds later.  No loaded value ever lands
    // in a register it has to carry across rounds: the compiler could only wait
    // for it by draining every load still streaming.
    auto slot_ok = [&](int u) { return u < u1 && u * kSub + l32 < p.topk; };  // sparse slot l32 exists
    // ring rows of sub-tile x
    auto idx_slot = [&](int x) -> MLA_LDS int32_t* { return ring_idx + (x & (kRingIdx - 1)) * 64; };
    auto pg_slot = [&](int x) -> MLA_LDS int32_t* { return ring_pg + (x & (kRingPg - 1)) * 64; };
    // Direct metadata loads into the rings (64 lanes each; lanes 32..63 repeat
    // 0..31): the indices of sub-tile x, the pages of sub-tile x's indices (its
    // indices must be visible).
    auto fetch_idx = [&](int x) {
      const int si = min(x * kSub + l32, p.topk - 1);
      buffer_load_lds4(idx_rs, (MLA_LDS void*)idx_slot(x), (uint32_t)si * 4u);
    };
    auto fetch_pg = [&](int x) {
      const int idx = idx_slot(x)[l32];
      const bool ok = slot_ok(x) && idx >= 0;
      buffer_load_lds4(bt_rs, (MLA_LDS void*)pg_slot(x), (uint32_t)(ok ? idx >> 6 : 0) * 4u);
    };
    // round u's share: part 0 the indices of sub-tile u + 8, part 1 the pages of
    // sub-tile u + 6
    auto meta_dma = [&](int u, int part) {
      if (part == 0)
        fetch_idx(u + 8);
      else
        fetch_pg(u + 6);
    };
    // prologue: the ring entries of sub-tiles u0 .. u0 + 5 (pages) and u0 .. u0 + 7
    // (indices); ends with a barrier after which they are visible
    // (Q's loads start here too: waves 0..3 issue them and only pass the
    // barriers, while waves 4..7 fetch the entries, two sub-tiles each, and
    // wait for them.)
    auto meta_fill = [&]() {
      if (wave_s < 4) {
        stage_q(0, buffer(u0 + 2));
        stage_q(1, buffer(u0 + 3));
        lds_barrier();
        lds_barrier();
      } else {
        const int x = wave_s - 4;
        fetch_idx(u0 + x);
        fetch_idx(u0 + x + 4);
        tile_barrier_drain();
        fetch_pg(u0 + x);
        if (x < 2) fetch_pg(u0 + x + 4);
        tile_barrier_drain();
      }
    };
    // attended mask of sub-tile u's 32 slots
    auto sparse_mask = [&](int u) -> uint32_t { return (uint32_t)__ballot(slot_ok(u) && idx_slot(u)[l32] >= 0); };
    // scores of sub-tile u with the slots this lane's row does not attend set to
    // -inf (this lane: row qrow, slots 16 tb + 4 h4 + e; tmask = sparse_mask(u),
    // read by the caller)
    auto mask_scores = [&](int u, f32x4& v, uint32_t tmask) {
      if (tmask != 0xFFFFFFFFu) {
        asm volatile("");  // a real branch: full sub-tiles skip the masking
        // tok0 is made opaque so that the compiler does not keep 4 token numbers
        // live across the loop
        int tok0 = 16 * tb + 4 * h4;
        asm volatile("" : "+v"(tok0));
        const uint32_t lmask = tmask >> tok0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ((lmask >> e) & 1u) != 0 ? v[e] : kNegInf;
      }
    };
    // ---- staging ------------------------------------------------------------------
    // Direct loads of sub-tile u: this thread's five (or four) 16-byte pieces,
    // gathered from per-slot token rows (the zero token, or an offset past the
    // pool, when a slot is not attended).  stage_begin reads the sub-tile's ring
    // entries; stage_load issues piece k.
    int st_tk[kLoads];  // token row (or -1) of each of this thread's pieces
    auto stage_begin = [&](int u) {
      {
        const int idx = idx_slot(u)[l32];
        const int pg = pg_slot(u)[l32];
        const int tok = (slot_ok(u) && idx >= 0) ? pg * kPage + (idx & 63) : -1;
        // each piece's token row, fetched from its slot's lane here, so that the
        // loads between the score MFMAs need no cross-lane (LDS) operation whose
        // wait would also wait for the K fragments in flight
        int to = tid;
        asm volatile("" : "+v"(to));
#pragma unroll
        for (int k = 0; k < kLoads; ++k) st_tk[k] = __shfl(tok, min(k * kDecThreads + to, kSlots - 1) / kTokenChunks);
      }
    };
    auto stage_load = [&](int k, MLA_LDS char* buf) {  // k < kLoads - 1, or waves 0..3
      MLA_LDS void* dst = (MLA_LDS void*)(buf + k * (kDecThreads * 16) + wave_s * 1024);
      {
        // the piece's token and source offset, recomputed from an opaque copy of
        // tid rather than kept live across the loop
        int to = tid;
        asm volatile("" : "+v"(to));
        const int s = min(k * kDecThreads + to, kSlots - 1);
        const int tt = s / kTokenChunks;
        const int tk = st_tk[k];
        const uint32_t chunk = (uint32_t)((s - tt * kTokenChunks) ^ tile_swizzle(tt)) * 16u;
        if constexpr (BUFG) {
          // MUBUF keeps the compiler's wait counts exact (a FLAT load into LDS
          // makes every later wait a full drain)
          const __amdgpu_buffer_rsrc_t pool_rs =
              __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, 0, p.pool_records, kBufferFlags);
          buffer_load_lds16(pool_rs, dst, tk >= 0 ? (uint32_t)tk * (uint32_t)kBf16TokenBytes + chunk : kPastPool);
        } else {
          const uint8_t* src = (tk >= 0 ? p.kv + (int64_t)tk * kBf16TokenBytes : g_zero_token) + chunk;
          global_load_lds16((const void*)src, dst);
        }
      }
    };
    auto stage_bf16 = [&](int u, MLA_LDS char* buf) {
      stage_begin(u);
#pragma unroll
      for (int k = 0; k < kLoads - 1; ++k) stage_load(k, buf);
      if (wave_s < 4) stage_load(kLoads - 1, buf);
    };
    // ---- operand reads ------------------------------------------------------------
    auto kread = [&](MLA_LDS char* kb, int kk) -> bf16x8 {
      return *(MLA_LDS bf16x8*)(kb + kofs[kk & 1] + (kk >> 1) * 128);
    };
    // V^T fragment: 32-column block ct of this wave's 64 columns, 16-token k-step s2
    auto vread = [&](MLA_LDS char* vb, int s2, int ct) -> bf16x8 {
      const int o = vofs[ct & 1] + 64 * ct + 16 * s2 * kBf16TokenBytes;
      const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + o));
      const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(vb + o + 4 * kBf16TokenBytes));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P fragment (B operand of PV): row block rb, k-step s2 of the sub-tile of parity par
    auto pread = [&](int par, int rb, int s2) -> bf16x8 {
      return *(MLA_LDS bf16x8*)(pbuf + par * kPHalf + ((rb * 2 + s2) * 64 + lane) * 16);
    };
    // row maximum over the lanes (h4 = 0..3) holding this lane's row
    auto row_max16 = [&](float v) -> float {
      v = fmaxf(v, __shfl_xor(v, 16));
      return fmaxf(v, __shfl_xor(v, 32));
    };

    // Reference maximum m_ref (log2 domain, per row): the row's maximum over the
    // split's first sub-tile + kRefLift, fixed for the whole split, so
    // P = 2^(x - m_ref) stays within [2^-126, 2^(kRefLift + kRefRoom)] for every
    // score within (kRefRoom, 126 - kRefLift) of that maximum, and O changes only
    // through MFMAs.  A score more than kRefRoom above m_ref (scores spread by
    // over ~60 natural-log units), or a finite score in a row whose first
    // sub-tile was fully masked, marks the pass as overflowed and the split is
    // recomputed from the start with the split's true row maximum as the
    // reference.
    float m_ref = kNegInf, m_seen = kNegInf, l_sum = 0.f;
    bool redo = false;
    int pass = 0;  // at most two: the second pass runs with the split's row maximum
    // K fragments read ahead of their score MFMA (the first ones before the
    // round's barrier)
    constexpr int kAhead = 4;
    constexpr int kPRead = 13;  // score MFMA after which the P fragments are read
    do {
      l_sum = 0.f;
      bool overflow = false;

      // ---- prologue ---------------------------------------------------------------
      // Q goes through the buffers of sub-tiles u0 + 2 and u0 + 3 before they
      // hold tiles: sub-tiles u0 and u0 + 1 and Q issued; u0 and Q landed; Q read;
      // then u0 + 2 issued into its buffer.  Then S of u0 and the reference.
      meta_fill();
      // Sub-tile u0 + 1 is loaded even when the split ends first (the zero
      // token keeps such loads in bounds; the buffer is not read), so every path
      // issues the same loads.
      stage_bf16(u0, buffer(u0));
      stage_bf16(u0 + 1, buffer(u0 + 1));
      // u0 and Q (waves 0..3, older) landed; u0 + 1 (5 or 4 loads per wave)
      // stays in flight
      if (wave_s < 4)
        barrier_keep<kLoads>();
      else
        barrier_keep<kLoads - 1>();
      read_q(buffer(u0 + 2), buffer(u0 + 3));
      lds_barrier();  // every wave has read Q before sub-tile u0 + 2 lands there
      // (loaded whether or not it exists, as u0 + 1; waited for with u0 + 1 at
      // the first round's closing wait)
      stage_bf16(u0 + 2, buffer(u0 + 2));
      // K fragments kk .. kk + kAhead - 1 of the next score step (rolling)
      bf16x8 kf[kAhead];
      f32x4 s;  // S^T of the sub-tile whose softmax comes next
      {
        MLA_LDS char* kb = buffer(u0);
#pragma unroll
        for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(kb, kk);
        s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk % kAhead], qf[kk], s, 0, 0, 0);
          if (kk + kAhead < 18) kf[kk % kAhead] = kread(kb, kk + kAhead);
        }
      }
      if (!redo) {
        // the reference of each row from sub-tile u0 (both token blocks of the row)
        f32x4 v = s;
        mask_scores(u0, v, sparse_mask(u0));
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        mx = row_max16(mx);
        if (h4 == 0) xrow[tb * 64 + qrow] = mx;
        lds_barrier();
        const float m0 = fmaxf(xrow[qrow], xrow[64 + qrow]) * p.scale_log2;
        m_ref = m0 == kNegInf ? kNegInf : m0 + kRefLift;
        // xrow is next written after the loop, behind at least one round's barrier
      }

      // (zeroed here, after the prologue's loads, not before them)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[rb][ct][e] = 0.f;
      // V^T fragments of the sub-tile whose PV comes next (read before the barrier
      // that precedes that PV)
      bf16x8 va[2][2];
      // One round u, entered after the barrier that ended round u - 1, with S(u)
      // in s (round u0: from the prologue), the first K fragments of sub-tile u in
      // kf, V^T of sub-tile u - 1 in va and P of sub-tile u - 1 in LDS:
      //   scores of sub-tile u (round u0: computed already), with the direct loads
      //   of sub-tile u + 3 between the MFMAs;
      //   O += P V of sub-tile u - 1, with the softmax of sub-tile u, its P write
      //   and the V^T reads of sub-tile u between the MFMAs;
      //   the first K fragments of sub-tile u + 1; one barrier.
      // So every MFMA operand a round needs after its barrier is in VGPRs or was
      // written before it, and the LDS and VALU work sits between MFMAs.  The
      // buffers are distinct, and saying so (restrict) lets the compiler keep the
      // direct loads in flight across the reads of kb and kn.
      // Compile-time knobs: kFirst (round u0); kIssue = 1 when sub-tile u + 3 is
      // known to exist (the main loop), -1 when that is decided at run time.
      // BF16 load accounting: a round that stages issues exactly kLoads vector
      // memory operations per wave (waves 0..3 five tile pieces, waves 4..7 four
      // and one metadata load), so its closing wait is one count for every wave.
      auto round = [&](auto first_tag, auto issue_tag, auto kself_tag, const int u,
                       MLA_LDS char* __restrict__ kb, MLA_LDS char* __restrict__ kn,
                       MLA_LDS char* __restrict__ nxt) __attribute__((always_inline)) {
        constexpr bool kFirst = decltype(first_tag)::value != 0;
        // this round reads its first K fragments itself (the round after u0,
        // whose sub-tile was still landing when round u0 ended)
        constexpr bool kSelfK = decltype(kself_tag)::value != 0;
        constexpr int kIssue = decltype(issue_tag)::value;
        const bool issue = kIssue == 1 || u + 3 < u1;  // sub-tile u + 3 exists (workgroup-uniform)
        __builtin_amdgcn_sched_barrier(0);
        // staging work placed after score MFMA kk
        auto stage_step = [&](int kk) __attribute__((always_inline)) {
          if (issue) {
            if (kk == 0) stage_begin(u + 3);
            if (kk % 3 == 1 && kk / 3 < kLoads - 1) stage_load(kk / 3, nxt);
            if (kk == 3 * (kLoads - 1) + 1) {
              if (wave_s < 4)
                stage_load(kLoads - 1, nxt);
              else  // waves 4, 5: metadata part 0; 6, 7: part 1
                meta_dma(u, (wave_s >> 1) & 1);
            }
          }
        };
        bf16x8 pp[2][2];  // P of sub-tile u - 1, read while the last score MFMAs run
        if constexpr (!kFirst) {
          if constexpr (kSelfK)
#pragma unroll
            for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(kb, kk);
          s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk % kAhead], qf[kk], s, 0, 0, 0);
            if (kk + kAhead < 18) kf[kk % kAhead] = kread(kb, kk + kAhead);
            if (kk == kPRead)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) pp[rb][s2] = pread((u - 1) & 1, rb, s2);
            stage_step(kk);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) stage_step(kk);
        }
        // softmax of sub-tile u: P = 2^(scale_log2 S - m_ref)
        auto softmax = [&]() __attribute__((always_inline)) {
          f32x4 v = s;
          mask_scores(u, v, sparse_mask(u));
          const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])) * p.scale_log2;
          m_seen = fmaxf(m_seen, mx);
          overflow |= (m_ref == kNegInf && mx != kNegInf) || mx > m_ref + kRefRoom;
          const float msafe = m_ref == kNegInf ? 0.f : m_ref;
          bf16x2 p01, p23;
          float pe[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], p.scale_log2, -msafe));
          l_sum += (pe[0] + pe[1]) + (pe[2] + pe[3]);
          p01.x = (__bf16)pe[0];
          p01.y = (__bf16)pe[1];
          p23.x = (__bf16)pe[2];
          p23.y = (__bf16)pe[3];
          *(MLA_LDS u32x2*)(pbuf + (u & 1) * kPHalf + pw_off) =
              u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
        };
        // PV(u - 1): O^T += V^T P^T (P of every wave, V^T of this wave's columns);
        // each V^T fragment is replaced by sub-tile u's once its two MFMAs issued
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            if constexpr (!kFirst) {
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][ct], pp[rb][s2], acc[rb][ct], 0, 0, 0);
            }
            va[s2][ct] = vread(kb, s2, ct);
            if (s2 == 0 && ct == 0) softmax();
            __builtin_amdgcn_sched_barrier(0);
          }
        // the first K fragments of sub-tile u + 1
        if constexpr (!kFirst)
          if (kIssue == 1 || u + 1 < u1)
#pragma unroll
            for (int kk = 0; kk < kAhead; ++kk) kf[kk] = kread(kn, kk);
        if (issue) {
          barrier_keep<kLoads>();  // the previous round's loads (sub-tile u + 2, metadata) have landed
        } else {
          tile_barrier_drain();
        }
      };
      constexpr int kStageAhead = 3;  // the sub-tile a round stages
      round(Tag<1>{}, Tag<-1>{}, Tag<0>{}, u0, buffer(u0), buffer(u0 + 1), buffer(u0 + kStageAhead));
      int u = u0 + 1;
      if (u < u1) {
        round(Tag<0>{}, Tag<-1>{}, Tag<1>{}, u, buffer(u), buffer(u + 1), buffer(u + kStageAhead));
        ++u;
      }
      // main loop: every round stages an existing sub-tile; then the last rounds
      for (; u + 3 < u1; ++u)
        round(Tag<0>{}, Tag<1>{}, Tag<0>{}, u, buffer(u), buffer(u + 1), buffer(u + kStageAhead));
      for (; u < u1; ++u)
        round(Tag<0>{}, Tag<-1>{}, Tag<0>{}, u, buffer(u), buffer(u + 1), buffer(u + kStageAhead));

      // PV of the last sub-tile
      {
        bf16x8 pp[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pp[rb][s2] = pread((u1 - 1) & 1, rb, s2);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s2][ct], pp[rb][s2], acc[rb][ct], 0, 0, 0);
      }

      // the restart must be taken by the whole workgroup (it contains barriers);
      // the vote is over every lane, so it is taken before the lane-0 store.
      // The same barrier publishes l and m_ref of each row for the epilogue
      // (l of a row: this lane's sum over its tokens, over the 4 lanes of the row
      // and the two token blocks); a restarted pass recomputes both.
      const bool wave_overflow = __ballot(overflow) != 0;
      if (lane == 0) wflag[wave_s] = wave_overflow ? 1 : 0;
      l_sum += __shfl_xor(l_sum, 16);
      l_sum += __shfl_xor(l_sum, 32);
      {
        int lo = lane;
        asm volatile("" : "+v"(lo));  // the row index is formed here, not kept live across the loop
        const int qr = 16 * r4 + (lo & 15);
        if (lo < 16) {
          xrow[tb * 64 + qr] = l_sum;
          if (tb == 0) xrow[128 + qr] = m_ref;
        }
      }
      __syncthreads();
      redo = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) redo |= wflag[i] != 0;
      redo = redo && pass == 0;
      ++pass;
      if (redo) {
        // the split's row maximum over every lane and token block holding the row
        // (no wave reads the rows' l and m_ref once a restart is decided)
        const float ms = row_max16(m_seen);
        if (h4 == 0) xrow[tb * 64 + qrow] = ms;
        __syncthreads();
        const float m0 = fmaxf(xrow[qrow], xrow[64 + qrow]);
        m_ref = m0 == kNegInf ? kNegInf : m0 + kRefLift;
        // (xrow and wflag are next written at the end of the restarted pass,
        // after its rounds' barriers)
      }
    } while (redo);

    // ---- epilogue -------------------------------------------------------------------
    // The normalised rows go through LDS (the free tile buffers, rows padded by
    // 16 bytes against bank conflicts) so that the global stores are whole
    // contiguous runs: the tile's rows are contiguous in o and in the split's
    // partial output, while each lane's accumulators hold 4 columns of 32
    // different rows (per-lane stores would write 32 scattered pieces each).
    const int nrows = min(p.R_stream - rt * kRowTile, kRowTile);  // rows of this tile that exist
    {
      // this lane's first output column; computed here (not hoisted out of the
      // stream loop, where it would hold registers the main loop needs)
      int lo = lane;
      asm volatile("" : "+v"(lo));
      const int col = 64 * wave_s + 4 * (lo >> 5);
      const int lrow = lo & 31;
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
          for (int ct = 0; ct < 2; ++ct)
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
          if (wave_s == 0 && h2 == 0 && rowj < p.R_stream) p.lse[row_base + rowj] = lse_v;
        } else {
          MLA_LDS char* prow = smem + rho * kOutRowF32 + col * 4;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& a = acc[rb][ct];
              *(MLA_LDS f32x4*)(prow + (ct * 32 + 8 * i) * 4) =
                  f32x4{a[4 * i] * inv, a[4 * i + 1] * inv, a[4 * i + 2] * inv, a[4 * i + 3] * inv};
            }
          if (wave_s == 0 && h2 == 0 && rowj < p.R_stream) {
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
      int to = tid;
      asm volatile("" : "+v"(to));
      if (final_out) {
        char* dst = (char*)(p.o + (row_base + rt * kRowTile) * kDV);
#pragma unroll
        for (int k = 0; k < kRowTile * kDV * 2 / 16 / kDecThreads; ++k) {
          const int c = k * kDecThreads + to;
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
          merge_split_tile<kDecThreads>(p, smem, kOutRowF32, stream, rt, sid, split_off[stream], nsplit, nrows, live,
                                        wflag, to);
        } else {
          char* dst = (char*)(p.part_o + ((int64_t)sid * p.R_stream + rt * kRowTile) * kDV);
#pragma unroll
          for (int k = 0; k < kRowTile * kDV * 4 / 16 / kDecThreads; ++k) {
            const int c = k * kDecThreads + to;
            const int row = c >> 7, off = (c & 127) * 16;
            if (row < nrows && ((live >> row) & 1u)) *(u32x4*)(dst + row * (kDV * 4) + off) = *(MLA_LDS u32x4*)(smem + row * kOutRowF32 + off);
          }
        }
      }
    }
    // the next piece reuses LDS; after the last one there is nothing to wait for
    if (stream < es && stream + 1 < p.n_streams) __syncthreads();
  }
  if (p.merge && p.topk == 0) zero_empty_streams<kDecThreads>(p, tid);
}

template <bool BUFG>
hipError_t launch_variant(const DecodeParams& p, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  auto kern = mla_decode_kernel<BUFG>;
  const hipError_t e = set_lds_limit((const void*)kern, kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.W * p.n_rt), dim3(kDecThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, bool is_fp8, hipStream_t stream) {
  const bool sparse = p.topk > 0;
  if (is_fp8) return launch_decode_fp8(p, stream);
  if (!sparse) return launch_decode_dense(p, stream);
  return p.pool_records != 0 ? launch_variant<true>(p, stream) : launch_variant<false>(p, stream);
}

}  // namespace mla
