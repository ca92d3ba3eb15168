// Shared definitions of the HIP library: sizes of the MLA latent, the paged
// cache layouts, the metadata layout and the kernel entry points the host API
// launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace mla {

constexpr int kDQK = 576;             // latent dims per token (K)
constexpr int kDV = 512;              // leading latent dims used as V
constexpr int kPage = 64;             // tokens per cache page
constexpr int kFp8Dims = 512;         // e4m3-coded dims of an FP8 token
constexpr int kFp8TokenBytes = 656;   // 512 codes + 4 fp32 scales + 64 bf16 RoPE dims
constexpr int kBf16TokenBytes = 1152;
constexpr int kTokenChunks = 72;      // 16-byte chunks of a bf16 token row

// Metadata: int32 words.
//   [0, 16)                         header (MH_* below)
//   [16, 16 + 8 W)                  per-worker schedule: begin_stream, begin_tile,
//                                   end_stream, end_tile (end exclusive), first_split,
//                                   the first piece's end tile, its stream's splits
//   [.., + n_streams + 1)           split_offset: first split id of each stream
//   [.., + n_streams + 1)           tile_first: first global tile of each stream
//   [.., + n_streams * row tiles)   arrival counters of the merging decode
//                                   (zeroed by the scheduler; each merge resets
//                                   its counter to 0)
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

inline __host__ __device__ int64_t meta_words(int W, int n_streams, int n_rt) {
  return kMetaHeader + (int64_t)kSchedStride * W + 2 * ((int64_t)n_streams + 1) + (int64_t)n_streams * n_rt;
}
inline __host__ __device__ int64_t meta_split_offset(int W) { return kMetaHeader + (int64_t)kSchedStride * W; }
inline __host__ __device__ int64_t meta_tile_first(int W, int n_streams) {
  return meta_split_offset(W) + (int64_t)n_streams + 1;
}
inline __host__ __device__ int64_t meta_arrive(int W, int n_streams) {
  return meta_tile_first(W, n_streams) + (int64_t)n_streams + 1;
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
  int merge;                 // 1: the last split of each (stream, row tile) merges the splits (no combine launch)
  int32_t* arrive;           // [n_streams * n_rt] arrival counters (in the metadata), used when merge = 1
};

// Splits a merging decode call merges in the decode kernel at most per stream.
constexpr int kMergeMaxSplits = 4;

// lse merge of one row's n <= NMAX split results (FlashMLA source walk-through,
// combine section): L = ln sum_j exp(lse_j), evaluated around the largest lse;
// o = sum_j exp(lse_j - L) o_j over 8 columns (v, v2: 4 each).  A split with
// lse = -inf (nothing attended) has weight 0 and its output is not used.
// Returns L (-inf when every split is empty, and then acc = 0).  The combine
// kernel and the merging decode kernel both use it, so they give the same bits.
template <int NMAX>
__device__ __forceinline__ float lse_merge(const float (&lj)[NMAX], const float4 (&v)[NMAX],
                                           const float4 (&v2)[NMAX], float4& acc, float4& acc2) {
  constexpr float kNegInf = -__builtin_huge_valf();
  acc = make_float4(0.f, 0.f, 0.f, 0.f);
  acc2 = acc;
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < NMAX; ++k) mx = fmaxf(mx, lj[k]);
  if (mx == kNegInf) return kNegInf;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NMAX; ++k) sum += lj[k] == kNegInf ? 0.f : __expf(lj[k] - mx);
  const float L = mx + __logf(sum);
#pragma unroll
  for (int k = 0; k < NMAX; ++k) {
    if (lj[k] == kNegInf) continue;
    // explicit fused multiply-adds: whether `acc += w * v` is contracted
    // depends on the surrounding code, and the two kernels must agree
    const float w = __expf(lj[k] - L);
    acc.x = __builtin_fmaf(w, v[k].x, acc.x);
    acc.y = __builtin_fmaf(w, v[k].y, acc.y);
    acc.z = __builtin_fmaf(w, v[k].z, acc.z);
    acc.w = __builtin_fmaf(w, v[k].w, acc.w);
    acc2.x = __builtin_fmaf(w, v2[k].x, acc2.x);
    acc2.y = __builtin_fmaf(w, v2[k].y, acc2.y);
    acc2.z = __builtin_fmaf(w, v2[k].z, acc2.z);
    acc2.w = __builtin_fmaf(w, v2[k].w, acc2.w);
  }
  return L;
}

// 8 fp32 -> 8 bf16 (RNE), packed.
__device__ __forceinline__ uint4 pack_bf16x8(const float4& a, const float4& b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t p0, p1, p2, p3;
  p0.x = (__bf16)a.x;
  p0.y = (__bf16)a.y;
  p1.x = (__bf16)a.z;
  p1.y = (__bf16)a.w;
  p2.x = (__bf16)b.x;
  p2.y = (__bf16)b.y;
  p3.x = (__bf16)b.z;
  p3.y = (__bf16)b.w;
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Raises a kernel's dynamic LDS limit on the current device, once per device
// (the attribute is a per-device setting; `done` holds one bit per device
// ordinal below 64, set after a successful call, and larger ordinals set it on
// every launch).  Concurrent first calls on one device both set it, which is
// harmless.
inline hipError_t set_lds_limit(const void* kern, int lds_bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

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
