// Host side of the C ABI (include/mla_decode.h): argument validation, sizing,
// workspace carving and kernel launches.  Validation happens before any HIP
// call, so a rejected call launches nothing and touches no device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "../../include/mla_decode.h"
#include "mla_common.hpp"

namespace {

thread_local char g_err[512] = "";
// bench hook: events recorded around the decode kernel (both set or both null)
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
// when the decode kernel merges the splits itself (mla_set_merge_mode)
thread_local int g_merge_mode = MLA_MERGE_OFF;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Smallest number of 64-token tiles a worker takes (the per-split cost term).
// A split costs its workgroups a fixed ~10 us (prologue, epilogue) and writes
// n_rt x 64 rows of fp32 partials that the combine reads back, so with more
// row tiles per stream a split must be longer to pay for itself.  Calibrated on
// decode calls whose total work is under two tiles per worker (with more work
// the rule does not bind): for 128- and 256-row streams 4 tiles beat 2 by 2-11 %
// (BF16 dense 27.7 -> 24.4 us, 27.9 -> 25.8, 32.4 -> 30.2; FP8 0-4 %) and 8
// (for 256 rows) was worse than 4; for 64-row streams 2 beat 4 by 1-11 %
// (c5-like FP8 sparse 24.1 vs 26.8 us); 1 was worse everywhere.  The cache type
// and topk did not change the best choice.
int min_tiles_for(int is_fp8, int topk, int n_rt) {
  (void)is_fp8;
  (void)topk;
  return n_rt >= 2 ? 4 : 2;
}

struct Shape {
  int n_streams, R, RT, n_rt;
};

// Whether a decode call merges its splits in the decode kernel (the last split
// of each row tile merges; no combine launch).  That needs every stream to have
// at most kMergeMaxSplits splits, which the host proves from what it knows:
// sparse streams have exactly T = ceil(topk / 64) tiles and the worker size
// q = max(ceil(N / W), m) is exact; a dense stream has at most max_blocks tiles
// (its block-table row covers it) and q >= m.  A stream of t tiles meets at
// most min(W, ceil(t / q) + 1) workers.
bool merge_ok(const Shape& s, int W, int topk, int max_blocks, int min_tiles, int mode) {
  if (mode != MLA_MERGE_ON) return false;
  int64_t tiles, q;
  if (topk > 0) {
    tiles = (topk + mla::kPage - 1) / mla::kPage;
    const int64_t N = (int64_t)s.n_streams * tiles;
    q = std::max<int64_t>(std::max<int64_t>((N + W - 1) / W, min_tiles), 1);
  } else {
    tiles = max_blocks;
    q = std::max(min_tiles, 1);
  }
  return std::min<int64_t>(W, (tiles + q - 1) / q + 1) <= mla::kMergeMaxSplits;
}

int shape_of(int B, int s_q, int h_q, int h_kv, int topk, Shape* s) {
  if (B < 1 || s_q < 1 || h_q < 1) return fail(MLA_ERR_INVALID_ARG, "B, s_q and h_q must be >= 1 (got %d, %d, %d)", B, s_q, h_q);
  if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", h_kv);
  if (topk < 0) return fail(MLA_ERR_INVALID_ARG, "topk must be >= 0 (got %d)", topk);
  const int64_t streams = topk > 0 ? (int64_t)B * s_q : (int64_t)B;
  const int64_t R = topk > 0 ? (int64_t)h_q : (int64_t)s_q * h_q;
  if (streams > (1 << 24) || R > (1 << 16)) return fail(MLA_ERR_UNSUPPORTED, "too many streams or rows per stream");
  s->n_streams = (int)streams;
  s->R = (int)R;
  s->RT = mla::kRowTile;
  s->n_rt = (s->R + s->RT - 1) / s->RT;
  return MLA_OK;
}

std::mutex g_cu_mu;
int g_cu_count[64] = {0};

int device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (dev >= 0 && dev < 64 && g_cu_count[dev] > 0) {
    *out = g_cu_count[dev];
    return MLA_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (dev >= 0 && dev < 64) g_cu_count[dev] = n;
  *out = n;
  return MLA_OK;
}

int resolve_workers(int num_workers, const Shape& s, int* W) {
  if (num_workers < 0) return fail(MLA_ERR_INVALID_ARG, "num_workers must be >= 0");
  if (num_workers > 0) {
    *W = num_workers;
    return MLA_OK;
  }
  int cus = 0;
  const int rc = device_cus(&cus);
  if (rc != MLA_OK) return rc;
  int w = cus / s.n_rt;
  if (w >= 8) w &= ~7;  // keep a worker's row tiles on one XCD
  *W = w < 1 ? 1 : w;
  return MLA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

void sizes(const Shape& s, int W, size_t* meta, size_t* part_o, size_t* ws) {
  const size_t max_splits = (size_t)W + (size_t)s.n_streams;
  *meta = (size_t)mla::meta_words(W, s.n_streams, s.n_rt) * sizeof(int32_t);
  *part_o = align_up(max_splits * (size_t)s.R * mla::kDV * sizeof(float));
  *ws = *part_o + align_up(max_splits * (size_t)s.R * sizeof(float));
}

// Sparse prefill workspace: the single request's length (int32), its identity
// page table (one int32 per 64-token piece of the sequence), the scheduler's
// metadata and the decode workspace, each 256-byte aligned.
struct PrefillLayout {
  size_t pages_off, meta_off, meta_bytes, ws_off, ws_bytes, total;
  int n_pages, W;
};

int prefill_layout(int s_q, int h_q, int h_kv, int64_t s_kv, int topk, int num_workers, PrefillLayout* L) {
  if (s_kv < 1 || s_kv > INT32_MAX - mla::kPage) return fail(MLA_ERR_INVALID_ARG, "s_kv must be in [1, 2^31 - 65]");
  if (topk < 1) return fail(MLA_ERR_INVALID_ARG, "sparse prefill needs topk >= 1 (got %d)", topk);
  Shape s;
  int rc = shape_of(1, s_q, h_q, h_kv, topk, &s);
  if (rc != MLA_OK) return rc;
  rc = resolve_workers(num_workers, s, &L->W);
  if (rc != MLA_OK) return rc;
  size_t part_o;
  sizes(s, L->W, &L->meta_bytes, &part_o, &L->ws_bytes);
  L->n_pages = (int)((s_kv + mla::kPage - 1) / mla::kPage);
  L->pages_off = kAlign;
  L->meta_off = align_up(L->pages_off + (size_t)L->n_pages * sizeof(int32_t));
  L->ws_off = align_up(L->meta_off + L->meta_bytes);
  L->total = L->ws_off + L->ws_bytes;
  return MLA_OK;
}

// Scratch of mla_decode_with_kvcache_noalloc: the split workspace (partial
// outputs and their lse) in a static device array, for callers that cannot
// allocate.  In host code `scratch` is only a stand-in for the symbol; its
// device address (one copy per GPU) comes from hipGetSymbolAddress, taken once
// per device on the entry point's first call there and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MLA_ERR_UNSUPPORTED, "device ordinal %d beyond 63", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

MLA_API const char* mla_last_error(void) { return g_err; }

MLA_API int mla_get_metadata_size(int B, int s_q, int h_q, int h_kv, int topk, int num_workers, size_t* metadata_bytes,
                                  size_t* workspace_bytes, int* num_workers_out) {
  g_err[0] = 0;
  if (!metadata_bytes || !workspace_bytes) return fail(MLA_ERR_INVALID_ARG, "null size output pointer");
  Shape s;
  int rc = shape_of(B, s_q, h_q, h_kv, topk, &s);
  if (rc != MLA_OK) return rc;
  int W = 0;
  rc = resolve_workers(num_workers, s, &W);
  if (rc != MLA_OK) return rc;
  size_t meta, part_o, ws;
  sizes(s, W, &meta, &part_o, &ws);
  *metadata_bytes = meta;
  *workspace_bytes = ws;
  if (num_workers_out) *num_workers_out = W;
  return MLA_OK;
}

MLA_API int mla_get_metadata(const int32_t* cache_seqlens, int B, int s_q, int h_q, int h_kv, int topk, int is_fp8,
                             int num_workers, int32_t* metadata, size_t metadata_bytes, void* stream) {
  g_err[0] = 0;
  if (!cache_seqlens || !metadata) return fail(MLA_ERR_INVALID_ARG, "null cache_seqlens or metadata");
  if (is_fp8 != 0 && is_fp8 != 1) return fail(MLA_ERR_INVALID_ARG, "is_fp8 must be 0 or 1");
  Shape s;
  int rc = shape_of(B, s_q, h_q, h_kv, topk, &s);
  if (rc != MLA_OK) return rc;
  int W = 0;
  rc = resolve_workers(num_workers, s, &W);
  if (rc != MLA_OK) return rc;
  size_t meta, part_o, ws;
  sizes(s, W, &meta, &part_o, &ws);
  if (metadata_bytes < meta)
    return fail(MLA_ERR_BUFFER_TOO_SMALL, "metadata needs %zu bytes, got %zu", meta, metadata_bytes);
  const hipError_t e = mla::launch_sched(cache_seqlens, B, s_q, h_q, topk, W, min_tiles_for(is_fp8, topk, s.n_rt),
                                         metadata, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "scheduler launch");
  return MLA_OK;
}

MLA_API int mla_decode_with_kvcache(const void* q, const void* kvcache, int64_t num_blocks, const int32_t* block_table,
                                    int max_blocks, const int32_t* cache_seqlens, int B, int s_q, int h_q, int h_kv,
                                    int d_qk, int d_v, float softmax_scale, int32_t* metadata,
                                    size_t metadata_bytes, int num_workers, const int32_t* indices, int topk,
                                    int is_fp8, int causal, void* workspace, size_t workspace_bytes, void* o,
                                    float* lse, void* stream) {
  g_err[0] = 0;
  if (!q || !kvcache || !block_table || !cache_seqlens || !metadata || !o || !lse || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (d_qk != mla::kDQK || d_v != mla::kDV)
    return fail(MLA_ERR_UNSUPPORTED, "only d_qk = 576 and d_v = 512 are supported (got %d, %d)", d_qk, d_v);
  if (num_blocks < 1 || max_blocks < 1) return fail(MLA_ERR_INVALID_ARG, "num_blocks and max_blocks must be >= 1");
  if (is_fp8 != 0 && is_fp8 != 1) return fail(MLA_ERR_INVALID_ARG, "is_fp8 must be 0 or 1");
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (causal && topk > 0)
    return fail(MLA_ERR_INVALID_ARG, "causal masking applies to dense decoding; index lists decide sparse visibility");
  if (topk > 0 && !indices) return fail(MLA_ERR_INVALID_ARG, "topk > 0 needs indices");
  if (topk == 0 && indices) return fail(MLA_ERR_INVALID_ARG, "indices given with topk = 0");
  if ((((uintptr_t)q) | ((uintptr_t)kvcache) | ((uintptr_t)o) | ((uintptr_t)workspace)) & 15)
    return fail(MLA_ERR_INVALID_ARG, "q, kvcache, o and workspace must be 16-byte aligned");
  Shape s;
  int rc = shape_of(B, s_q, h_q, h_kv, topk, &s);
  if (rc != MLA_OK) return rc;
  int W = 0;
  rc = resolve_workers(num_workers, s, &W);
  if (rc != MLA_OK) return rc;
  size_t meta, part_o, ws;
  sizes(s, W, &meta, &part_o, &ws);
  if (metadata_bytes < meta)
    return fail(MLA_ERR_BUFFER_TOO_SMALL, "metadata needs %zu bytes, got %zu", meta, metadata_bytes);
  if (workspace_bytes < ws)
    return fail(MLA_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", ws, workspace_bytes);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)mla::kDQK);

  mla::DecodeParams p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint8_t*)kvcache;
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.indices = indices;
  p.meta = metadata;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + part_o);
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.max_blocks = max_blocks;
  p.topk = topk;
  p.B = B;
  p.s_q = s_q;
  p.h_q = h_q;
  p.R_stream = s.R;
  p.n_streams = s.n_streams;
  p.n_rt = s.n_rt;
  p.W = W;
  p.causal = causal;
  p.scale_log2 = scale * 1.4426950408889634f;
  const uint64_t pool_bytes = (uint64_t)num_blocks * mla::kPage * (is_fp8 ? mla::kFp8TokenBytes : mla::kBf16TokenBytes);
  p.pool_records = pool_bytes <= 0xFFFFFF00ull ? (uint32_t)pool_bytes : 0u;
  p.merge = merge_ok(s, W, topk, max_blocks, min_tiles_for(is_fp8, topk, s.n_rt), g_merge_mode) ? 1 : 0;
  p.arrive = metadata + mla::meta_arrive(W, s.n_streams);
  hipError_t e = hipSuccess;
  if (g_ev_start && (e = hipEventRecord(g_ev_start, (hipStream_t)stream)) != hipSuccess)
    return hip_fail(e, "decode start event");
  e = mla::launch_decode(p, is_fp8 != 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (g_ev_stop && (e = hipEventRecord(g_ev_stop, (hipStream_t)stream)) != hipSuccess)
    return hip_fail(e, "decode stop event");
  if (!p.merge) {
    e = mla::launch_combine(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return MLA_OK;
}

MLA_API int mla_set_merge_mode(int mode) {
  g_err[0] = 0;
  if (mode != MLA_MERGE_OFF && mode != MLA_MERGE_ON)
    return fail(MLA_ERR_INVALID_ARG, "merge mode must be %d or %d (got %d)", MLA_MERGE_OFF, MLA_MERGE_ON, mode);
  g_merge_mode = mode;
  return MLA_OK;
}

MLA_API int mla_decode_with_kvcache_noalloc(const void* q, const void* kvcache, int64_t num_blocks,
                                            const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                                            int B, int s_q, int h_q, int h_kv, int d_qk, int d_v, float softmax_scale,
                                            int32_t* metadata, size_t metadata_bytes, int num_workers,
                                            const int32_t* indices, int topk, int is_fp8, int causal, void* o,
                                            float* lse, void* stream) {
  g_err[0] = 0;
  Shape s;
  int rc = shape_of(B, s_q, h_q, h_kv, topk, &s);
  if (rc != MLA_OK) return rc;
  int W = 0;
  rc = resolve_workers(num_workers, s, &W);
  if (rc != MLA_OK) return rc;
  size_t meta, part_o, ws;
  sizes(s, W, &meta, &part_o, &ws);
  if (ws > kScratchBytes)
    return fail(MLA_ERR_UNSUPPORTED, "this shape needs %zu bytes of split workspace; the static scratch holds %zu", ws,
                kScratchBytes);
  void* ptr = nullptr;
  rc = scratch_address(&ptr);
  if (rc != MLA_OK) return rc;
  return mla_decode_with_kvcache(q, kvcache, num_blocks, block_table, max_blocks, cache_seqlens, B, s_q, h_q, h_kv,
                                 d_qk, d_v, softmax_scale, metadata, metadata_bytes, W, indices, topk, is_fp8, causal,
                                 ptr, kScratchBytes, o, lse, stream);
}

MLA_API int mla_set_decode_kernel_events(void* start, void* stop) {
  g_err[0] = 0;
  if ((start == nullptr) != (stop == nullptr)) return fail(MLA_ERR_INVALID_ARG, "set both events or neither");
  g_ev_start = (hipEvent_t)start;
  g_ev_stop = (hipEvent_t)stop;
  return MLA_OK;
}

MLA_API int mla_debug_dequant_fp8(const uint8_t* tokens, int64_t n, void* out, void* stream) {
  g_err[0] = 0;
  if (!tokens || !out) return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "n must be >= 0");
  if ((((uintptr_t)tokens) | ((uintptr_t)out)) & 15) return fail(MLA_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  if (n == 0) return MLA_OK;
  const hipError_t e = mla::launch_debug_dequant(tokens, n, (uint16_t*)out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return MLA_OK;
}

MLA_API int mla_sparse_prefill_workspace_size(int s_q, int h_q, int h_kv, int64_t s_kv, int topk, int num_workers,
                                              size_t* workspace_bytes, int* num_workers_out) {
  g_err[0] = 0;
  if (!workspace_bytes) return fail(MLA_ERR_INVALID_ARG, "null size output pointer");
  PrefillLayout L;
  const int rc = prefill_layout(s_q, h_q, h_kv, s_kv, topk, num_workers, &L);
  if (rc != MLA_OK) return rc;
  *workspace_bytes = L.total;
  if (num_workers_out) *num_workers_out = L.W;
  return MLA_OK;
}

MLA_API int mla_sparse_prefill(const void* q, const void* kv, int64_t s_kv, const int32_t* indices, int s_q, int h_q,
                               int h_kv, int topk, int d_qk, int d_v, float softmax_scale, int num_workers,
                               void* workspace, size_t workspace_bytes, void* o, float* lse, void* stream) {
  g_err[0] = 0;
  if (!q || !kv || !indices || !workspace || !o || !lse) return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (d_qk != mla::kDQK || d_v != mla::kDV)
    return fail(MLA_ERR_UNSUPPORTED, "only d_qk = 576 and d_v = 512 are supported (got %d, %d)", d_qk, d_v);
  if ((((uintptr_t)q) | ((uintptr_t)kv) | ((uintptr_t)o) | ((uintptr_t)workspace)) & 15)
    return fail(MLA_ERR_INVALID_ARG, "q, kv, o and workspace must be 16-byte aligned");
  PrefillLayout L;
  int rc = prefill_layout(s_q, h_q, h_kv, s_kv, topk, num_workers, &L);
  if (rc != MLA_OK) return rc;
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", L.total, workspace_bytes);
  char* ws = (char*)workspace;
  int32_t* seqlen = (int32_t*)ws;
  int32_t* pages = (int32_t*)(ws + L.pages_off);
  int32_t* meta = (int32_t*)(ws + L.meta_off);
  hipError_t e = mla::launch_prefill_setup(seqlen, pages, L.n_pages, (int)s_kv, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill set-up launch");
  e = mla::launch_sched(seqlen, 1, s_q, h_q, topk, L.W, min_tiles_for(0, topk, (h_q + mla::kRowTile - 1) / mla::kRowTile),
                        meta, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "scheduler launch");
  return mla_decode_with_kvcache(q, kv, L.n_pages, pages, L.n_pages, seqlen, 1, s_q, h_q, h_kv, d_qk, d_v,
                                 softmax_scale, meta, L.meta_bytes, L.W, indices, topk, 0, 0, ws + L.ws_off,
                                 L.ws_bytes, o, lse, stream);
}

}  // extern "C"
