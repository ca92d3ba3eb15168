// Scheduler kernel: spreads the decode step's (stream, KV tile range) work
// evenly over W workers ahead of time, so the decode kernel only follows a
// precomputed plan (FlashMLA source walk-through, scheduling section: a small
// kernel divides (request, KV block range) units among all compute units before
// the main kernel runs; long sequences become several splits).
//
// Rule (deterministic, integer only):
//   streams: dense -> one per request with ceil(seqlen_b / 64) tiles;
//            sparse -> one per (request, query token) with ceil(topk / 64) tiles;
//   N = total tiles, q = max(ceil(N / W), min_tiles, 1);
//   worker w owns global tiles [w q, min((w + 1) q, N)) of the streams laid end
//   to end; each stream's splits are the workers that meet it, in worker order.
// One workgroup of 256 threads: chunked prefix sums (a shuffle scan across the
// threads' chunk sums) over the streams, then one binary search per worker.  Up to kLdsStreams streams the prefix arrays live in
// LDS (the searches then cost no global round trips); beyond that they are
// built in place in the metadata buffer.
#include "mla_common.hpp"

namespace mla {

namespace {

constexpr int kSchedThreads = 256;
constexpr int kLdsStreams = 8192;

__device__ __forceinline__ int64_t stream_tiles(const int32_t* seqlens, int topk, int i) {
  const int64_t len = topk > 0 ? (int64_t)topk : (int64_t)seqlens[i];
  return len > 0 ? (len + kPage - 1) / kPage : 0;
}

// Exclusive scan of one value per thread over the workgroup; every thread gets
// its exclusive prefix and the total.  Wave-level shuffles, then the four wave
// totals through LDS.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* wave_sums, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wave_sums[wave] = inc;
  __syncthreads();
  int64_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    const int64_t ws = wave_sums[w];
    if (w < wave) before += ws;
    total += ws;
  }
  __syncthreads();  // wave_sums is reused by the next scan
  return before + inc - v;
}

// First index in [0, n) with a[idx] > x (n if none); a non-decreasing.
__device__ int upper_bound(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] > x)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

__global__ __launch_bounds__(kSchedThreads) void mla_sched_kernel(const int32_t* __restrict__ seqlens, int B, int s_q,
                                                                  int h_q, int topk, int W, int min_tiles,
                                                                  int32_t* __restrict__ meta) {
  __shared__ int64_t wave_sums[kSchedThreads / 64];
  __shared__ int32_t lds_first[kLdsStreams + 1], lds_split[kLdsStreams + 1], lds_tiles[kLdsStreams];
  const int tid = threadIdx.x;
  const int n = topk > 0 ? B * s_q : B;
  int32_t* sched = meta + kMetaHeader;
  int32_t* g_split = meta + meta_split_offset(W);
  int32_t* g_first = meta + meta_tile_first(W, n);
  const bool in_lds = n <= kLdsStreams;
  int32_t* split_off = in_lds ? (int32_t*)lds_split : g_split;
  int32_t* first = in_lds ? (int32_t*)lds_first : g_first;

  const int per = (n + kSchedThreads - 1) / kSchedThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);

  // each stream's tile count, read from memory once (kept in LDS when it fits)
  auto tiles_of = [&](int i) -> int64_t { return in_lds ? (int64_t)lds_tiles[i] : stream_tiles(seqlens, topk, i); };

  // tile prefix sums
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) {
    const int64_t t = stream_tiles(seqlens, topk, i);
    if (in_lds) lds_tiles[i] = (int32_t)t;
    sum += t;
  }
  int64_t N;
  int64_t acc = block_exclusive_scan(sum, wave_sums, N);
  for (int i = lo; i < hi; ++i) {
    first[i] = (int32_t)acc;
    acc += tiles_of(i);
  }
  if (tid == 0) first[n] = (int32_t)N;
  int64_t q = (N + W - 1) / W;
  if (q < min_tiles) q = min_tiles;
  if (q < 1) q = 1;

  // splits per stream = workers meeting it
  sum = 0;
  for (int i = lo; i < hi; ++i) {
    const int64_t t = tiles_of(i);
    sum += t == 0 ? 0 : ((int64_t)first[i] + t - 1) / q - (int64_t)first[i] / q + 1;
  }
  int64_t total_splits;
  acc = block_exclusive_scan(sum, wave_sums, total_splits);
  for (int i = lo; i < hi; ++i) {
    split_off[i] = (int32_t)acc;
    const int64_t t = tiles_of(i);
    acc += t == 0 ? 0 : ((int64_t)first[i] + t - 1) / q - (int64_t)first[i] / q + 1;
  }
  if (tid == 0) split_off[n] = (int32_t)total_splits;
  __syncthreads();

  // per-worker ranges
  for (int w = tid; w < W; w += kSchedThreads) {
    int32_t* e = sched + (int64_t)w * kSchedStride;
    const int64_t wlo = (int64_t)w * q;
    int64_t whi = (int64_t)(w + 1) * q;
    if (whi > N) whi = N;
    int32_t v[kSchedStride] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (wlo >= N) {
      v[0] = v[2] = n;
    } else {
      const int bs = upper_bound(first, n + 1, wlo) - 1;
      const int es = upper_bound(first + 1, n, whi);
      v[0] = bs;
      v[1] = (int32_t)(wlo - first[bs]);
      v[2] = es;
      v[3] = es < n ? (int32_t)(whi - first[es]) : 0;
      v[4] = (int32_t)(split_off[bs] + (w - (int64_t)first[bs] / q));
      // the first piece's end tile and its stream's split count, so that the
      // decode kernel starts its first piece from this entry alone
      v[5] = es == bs ? v[3] : first[bs + 1] - first[bs];
      v[6] = split_off[bs + 1] - split_off[bs];
    }
    for (int k = 0; k < kSchedStride; ++k) e[k] = v[k];
  }
  if (in_lds)
    for (int i = tid; i <= n; i += kSchedThreads) {
      g_first[i] = first[i];
      g_split[i] = split_off[i];
    }
  // arrival counters of merging decode calls start at zero
  {
    const int R = topk > 0 ? h_q : s_q * h_q;
    const int64_t n_cnt = (int64_t)n * ((R + kRowTile - 1) / kRowTile);
    int32_t* arrive = meta + meta_arrive(W, n);
    for (int64_t i = tid; i < n_cnt; i += kSchedThreads) arrive[i] = 0;
  }
  if (tid == 0) {
    int32_t h[kMetaHeader] = {0};
    h[MH_MAGIC] = kMetaMagic;
    h[MH_NSTREAMS] = n;
    h[MH_W] = W;
    h[MH_Q] = (int32_t)q;
    h[MH_N] = (int32_t)N;
    h[MH_SPLITS] = (int32_t)total_splits;
    h[MH_RSTREAM] = topk > 0 ? h_q : s_q * h_q;
    h[MH_MINTILES] = min_tiles;
    h[MH_TOPK] = topk;
    h[MH_B] = B;
    h[MH_SQ] = s_q;
    h[MH_HQ] = h_q;
    for (int k = 0; k < kMetaHeader; ++k) meta[k] = h[k];
  }
}

}  // namespace

hipError_t launch_sched(const int32_t* seqlens, int B, int s_q, int h_q, int topk, int W, int min_tiles, int32_t* meta,
                        hipStream_t stream) {
  hipLaunchKernelGGL(mla_sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, seqlens, B, s_q, h_q, topk, W, min_tiles,
                     meta);
  return hipGetLastError();
}

}  // namespace mla
