// Shared definitions of the HIP library: sizes of the MLA latent, the paged
// cache layouts, the metadata layout and the kernel entry points the host API
// launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDQK = 576;             // latent dims per token (K)
constexpr int kDV = 512;              // leading latent dims used as V
constexpr int kPage = 64;             // tokens per cache page
constexpr int kFp8Dims = 512;         // e4m3-coded dims of an FP8 token
constexpr int kFp8TokenBytes = 656;   // 512 codes + 4 fp32 scales + 64 bf16 RoPE dims
constexpr int kBf16TokenBytes = 1152;
constexpr int kTokenChunks = 72;      // 16-byte chunks of a bf16 token row
constexpr int kTileBytes = kPage * kBf16TokenBytes;  // one page as bf16 in LDS

constexpr int kWaveRows = 32;  // query rows of one wave pair
constexpr int kThreads = 256;  // 4 waves

// Metadata: int32 words.
//   [0, 16)                         header (MH_* below)
//   [16, 16 + 8 W)                  per-worker schedule: begin_stream, begin_tile,
//                                   end_stream, end_tile (end exclusive), first_split,
//                                   the first piece's end tile, its stream's splits
//   [.., + n_streams + 1)           split_offset: first split id of each stream
//   [.., + n_streams + 1)           tile_first: first global tile of each stream
constexpr int kMetaHeader = 16;
constexpr int kSchedStride = 8;
constexpr int32_t kMetaMagic = 0x4D4C4131;
enum MetaHeader {
  MH_MAGIC = 0,
  MH_NSTREAMS,
  MH_W,
  MH_Q,        // tiles per worker
  MH_N,        // total tiles
  MH_SPLITS,   // total splits
  MH_RSTREAM,  // query rows per stream
  MH_MINTILES,
  MH_TOPK,
  MH_B,
  MH_SQ,
  MH_HQ,
};

inline __host__ __device__ int64_t meta_words(int W, int n_streams) {
  return kMetaHeader + (int64_t)kSchedStride * W + 2 * ((int64_t)n_streams + 1);
}
inline __host__ __device__ int64_t meta_split_offset(int W) { return kMetaHeader + (int64_t)kSchedStride * W; }
inline __host__ __device__ int64_t meta_tile_first(int W, int n_streams) {
  return meta_split_offset(W) + (int64_t)n_streams + 1;
}

// Query rows per decode workgroup (two row blocks of 32); a stream with more
// rows is covered by several row tiles that read the same KV range.
constexpr int kRowTile = 64;

struct DecodeParams {
  const uint16_t* q;         // bf16 [B, s_q, h_q, 576]
  const uint8_t* kv;         // cache bytes
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;    // [B, s_q, topk] or null
  const int32_t* meta;
  float* part_o;             // [max_splits, R_stream, 512]
  float* part_lse;           // [max_splits, R_stream]
  uint16_t* o;               // bf16 [B, s_q, h_q, 512]
  float* lse;                // [B, s_q, h_q]
  int max_blocks;
  int topk;
  int B, s_q, h_q;
  int R_stream;              // query rows per stream
  int n_streams;
  int n_rt;                  // row tiles (workgroups) per worker
  int W;                     // workers
  int causal;                // dense: query token s of s_q sees positions <= seqlen - s_q + s
  float scale_log2;          // softmax_scale * log2(e)
  uint32_t pool_records;     // sparse BF16: KV pool bytes when at most 0xFFFFFF00 (MUBUF gathers), else 0
};

// Launchers (each in its own .hip file).
hipError_t launch_sched(const int32_t* seqlens, int B, int s_q, int h_q, int topk, int W, int min_tiles,
                        int32_t* meta, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, bool is_fp8, hipStream_t stream);
hipError_t launch_decode_dense(const DecodeParams& p, hipStream_t stream);  // dense BF16 cache
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream);    // FP8 caches, dense and sparse
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);
hipError_t launch_prefill_setup(int32_t* seqlen, int32_t* pages, int n_pages, int s_kv, hipStream_t stream);
hipError_t launch_debug_dequant(const uint8_t* tokens, int64_t n, uint16_t* out, hipStream_t stream);

}  // namespace mla
