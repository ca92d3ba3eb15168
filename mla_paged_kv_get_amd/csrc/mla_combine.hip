// Combine kernel: merges the splits of each sequence by their lse (FlashMLA
// source walk-through, combine section: each split leaves a partial output and
// lse, and the combine kernel uses lse to fold them into the final result):
//   L = ln sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i,  lse = L.
// Streams with a single split were finished by the decode kernel; streams with
// no tiles (seqlen 0) get o = 0 and lse = -inf.
//
// One thread per (query row, 8 columns): it reads the row's split lse values
// (the same addresses for all 64 threads of a row, so one request per wave)
// together with its split outputs, 8 or 16 splits at a time, and forms L and
// the weights itself, so a workgroup pays one memory round trip per batch of
// splits instead of one per row it visits: one in all for up to 8 or 16
// splits, and an online merge over batches beyond that.
#include <algorithm>

#include "mla_common.hpp"

namespace mla {

namespace {

constexpr int kCombineThreads = 256;  // four rows x 64 threads (8 columns each)

// One thread's 8 columns of one row of the stream.
template <int kCombineFused>
__device__ __forceinline__ void combine_row(const DecodeParams& p, int stream, int s0, int n, int row) {
  const int c = (threadIdx.x & 63) * 8;
  const int64_t row_base = (int64_t)stream * p.R_stream;
  constexpr float kNegInf = -__builtin_huge_valf();
  const float* lse_col = p.part_lse + (int64_t)s0 * p.R_stream + row;  // split j at j * R_stream
  const float* po = p.part_o + ((int64_t)s0 * p.R_stream + row) * kDV + c;
  const int64_t stride = (int64_t)p.R_stream * kDV;

  auto write_out = [&](const float4& acc, const float4& acc2, float L) {
    *(uint4*)(p.o + (row_base + row) * kDV + c) = pack_bf16x8(acc, acc2);
    if (c == 0) p.lse[row_base + row] = L;
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acc2 = acc;

  if (n <= kCombineFused) {
    // Every split's output is loaded together with the lse values, before its
    // weight is known (one memory round trip).
    float lj[kCombineFused];
    float4 v[kCombineFused], v2[kCombineFused];
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) {
      lj[k] = k < n ? lse_col[(int64_t)k * p.R_stream] : kNegInf;
      v[k] = k < n ? *(const float4*)(po + k * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
      v2[k] = k < n ? *(const float4*)(po + k * stride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float L = lse_merge<kCombineFused>(lj, v, v2, acc, acc2);
    write_out(acc, acc2, L);
    return;
  }

  // More splits: one pass over them, kCombineFused at a time (lse values and
  // outputs loaded together, so one memory round trip per batch), merged
  // online: m is the largest lse so far, s = sum_j exp(lse_j - m) and
  // acc = sum_j exp(lse_j - m) o_j, both rescaled when m grows; then
  // L = m + ln s and o = acc / s.  (Loading the lse values one split after
  // another in a loop of their own made every split a round trip: a stream of
  // 32 splits took ~40 us.)
  float m = kNegInf, s = 0.f;
  for (int j0 = 0; j0 < n; j0 += kCombineFused) {
    float lj[kCombineFused];
    float4 v[kCombineFused], v2[kCombineFused];
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) {
      const int j = j0 + k;
      lj[k] = j < n ? lse_col[(int64_t)j * p.R_stream] : kNegInf;
      v[k] = j < n ? *(const float4*)(po + j * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
      v2[k] = j < n ? *(const float4*)(po + j * stride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = kNegInf;
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) bm = fmaxf(bm, lj[k]);
    if (bm == kNegInf) continue;  // every split of the batch is empty
    const float nm = fmaxf(m, bm);
    const float r = m == kNegInf ? 0.f : __expf(m - nm);
    s *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
    acc2.x *= r;
    acc2.y *= r;
    acc2.z *= r;
    acc2.w *= r;
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) {
      // an empty split (lse = -inf) carries weight 0; its output was not
      // written and is not used
      if (lj[k] == kNegInf) continue;
      const float w = __expf(lj[k] - nm);
      s += w;
      acc.x += w * v[k].x;
      acc.y += w * v[k].y;
      acc.z += w * v[k].z;
      acc.w += w * v[k].w;
      acc2.x += w * v2[k].x;
      acc2.y += w * v2[k].y;
      acc2.z += w * v2[k].z;
      acc2.w += w * v2[k].w;
    }
    m = nm;
  }
  const float L = m == kNegInf ? kNegInf : m + __logf(s);
  if (m != kNegInf) {
    const float inv = 1.f / s;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
    acc2.x *= inv;
    acc2.y *= inv;
    acc2.z *= inv;
    acc2.w *= inv;
  }
  write_out(acc, acc2, L);
}

// kCombineFused: up to this many splits, the lse values and the outputs are
// loaded together (8 or 16; the wider variant holds more VGPRs, so fewer waves
// fit on a CU, and the host uses it only when streams have many splits).
// kLoop: the grid is capped and each workgroup takes several groups of rows.
template <int kCombineFused, bool kLoop>
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(DecodeParams p) {
  const int stream = blockIdx.x;
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int s0 = split_off[stream];
  const int n = split_off[stream + 1] - s0;
  if (n == 1) return;  // finished by the decode kernel
  if constexpr (kLoop) {
    // a capped grid: this workgroup's share of the stream's groups of 4 rows
    const int groups = (p.R_stream + 3) / 4;
    const int per = (groups + (int)gridDim.y - 1) / (int)gridDim.y;
    const int g1 = min(groups, ((int)blockIdx.y + 1) * per);
    for (int g = (int)blockIdx.y * per; g < g1; ++g) {
      const int row = g * 4 + (threadIdx.x >> 6);
      if (row < p.R_stream) combine_row<kCombineFused>(p, stream, s0, n, row);
    }
  } else {
    const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (row < p.R_stream) combine_row<kCombineFused>(p, stream, s0, n, row);
  }
}

// Streams cut into many splits (a long request alone, say): one workgroup per
// row, its four waves each merging every fourth split of the row online in
// batches of 16 (lse values and outputs loaded together), then wave 0 merging
// the four partial results through LDS.  With one workgroup per 4 rows and every
// split of a row in one thread, a 131072-token request's 128 splits made 32
// workgroups of 8 dependent round trips each (18 us).
constexpr int kWideBatch = 16;
__global__ __launch_bounds__(kCombineThreads) void mla_combine_wide_kernel(DecodeParams p) {
  __shared__ float part_m[4], part_s[4];
  __shared__ float4 part_acc[4][2][64];
  const int stream = blockIdx.x, row = blockIdx.y;
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int s0 = split_off[stream];
  const int n = split_off[stream + 1] - s0;
  if (n == 1) return;  // finished by the decode kernel
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (n <= kWideBatch) {
    // few splits after all: wave 0 merges them in one pass, with the same
    // arithmetic as every other merge of up to 16 splits
    if (g == 0) combine_row<kWideBatch>(p, stream, s0, n, row);
    return;
  }
  constexpr float kNegInf = -__builtin_huge_valf();
  const int c = lane * 8;
  const float* lse_col = p.part_lse + (int64_t)s0 * p.R_stream + row;
  const float* po = p.part_o + ((int64_t)s0 * p.R_stream + row) * kDV + c;
  const int64_t stride = (int64_t)p.R_stream * kDV;
  float m = kNegInf, s = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acc2 = acc;
  for (int j0 = g; j0 < n; j0 += 4 * kWideBatch) {
    float lj[kWideBatch];
    float4 v[kWideBatch], v2[kWideBatch];
#pragma unroll
    for (int k = 0; k < kWideBatch; ++k) {
      const int j = j0 + 4 * k;
      lj[k] = j < n ? lse_col[(int64_t)j * p.R_stream] : kNegInf;
      v[k] = j < n ? *(const float4*)(po + j * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
      v2[k] = j < n ? *(const float4*)(po + j * stride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = kNegInf;
#pragma unroll
    for (int k = 0; k < kWideBatch; ++k) bm = fmaxf(bm, lj[k]);
    if (bm == kNegInf) continue;
    const float nm = fmaxf(m, bm);
    const float r = m == kNegInf ? 0.f : __expf(m - nm);
    s *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
    acc2.x *= r;
    acc2.y *= r;
    acc2.z *= r;
    acc2.w *= r;
#pragma unroll
    for (int k = 0; k < kWideBatch; ++k) {
      if (lj[k] == kNegInf) continue;  // an empty split: output not written
      const float w = __expf(lj[k] - nm);
      s += w;
      acc.x += w * v[k].x;
      acc.y += w * v[k].y;
      acc.z += w * v[k].z;
      acc.w += w * v[k].w;
      acc2.x += w * v2[k].x;
      acc2.y += w * v2[k].y;
      acc2.z += w * v2[k].z;
      acc2.w += w * v2[k].w;
    }
    m = nm;
  }
  if (lane == 0) {
    part_m[g] = m;
    part_s[g] = s;
  }
  part_acc[g][0][lane] = acc;
  part_acc[g][1][lane] = acc2;
  __syncthreads();
  if (g != 0) return;
  float M = kNegInf;
#pragma unroll
  for (int q = 0; q < 4; ++q) M = fmaxf(M, part_m[q]);
  float S = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f), o2 = o;
  if (M != kNegInf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (part_m[q] == kNegInf) continue;
      const float w = __expf(part_m[q] - M);
      S += w * part_s[q];
      const float4 a = part_acc[q][0][lane], b = part_acc[q][1][lane];
      o.x += w * a.x;
      o.y += w * a.y;
      o.z += w * a.z;
      o.w += w * a.w;
      o2.x += w * b.x;
      o2.y += w * b.y;
      o2.z += w * b.z;
      o2.w += w * b.w;
    }
    const float inv = 1.f / S;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    o2.x *= inv;
    o2.y *= inv;
    o2.z *= inv;
    o2.w *= inv;
  }
  const float L = M == kNegInf ? kNegInf : M + __logf(S);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 a, b, d, e;
  a.x = (__bf16)o.x;
  a.y = (__bf16)o.y;
  b.x = (__bf16)o.z;
  b.y = (__bf16)o.w;
  d.x = (__bf16)o2.x;
  d.y = (__bf16)o2.y;
  e.x = (__bf16)o2.z;
  e.y = (__bf16)o2.w;
  const int64_t row_base = (int64_t)stream * p.R_stream;
  *(uint4*)(p.o + (row_base + row) * kDV + c) =
      make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, d),
                 __builtin_bit_cast(uint32_t, e));
  if (lane == 0) p.lse[row_base + row] = L;
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  // One workgroup per (stream, 4 rows), unless that is more than eight passes of
  // the chip (many streams, e.g. sparse prefill, most with one split and their
  // workgroups returning at once): then about 2048 workgroups, each looping
  // over up to four of a stream's row groups (prefill combine 15.9 -> 5.6 us;
  // with few streams the loop measured slower, so it is not used there).
  const int groups = (p.R_stream + 3) / 4;
  const bool cap = (int64_t)p.n_streams * groups > 16384;
  const int gy = cap ? std::max((groups + 3) / 4, std::min(groups, (2048 + p.n_streams - 1) / p.n_streams)) : groups;
  const dim3 grid(p.n_streams, gy);
  // more than 8 workers per stream: streams are likely cut into more than 8
  // splits; more than 32: one workgroup per row, its waves sharing the splits
  // (a 131072-token request alone: decode call 68.2 -> 58.5 us; with 16 splits
  // per stream the one-row workgroups measured 0.9 us slower than one batch)
  if (p.W > 32 * p.n_streams && !cap) {
    hipLaunchKernelGGL(mla_combine_wide_kernel, dim3(p.n_streams, p.R_stream), dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
  }
  const bool wide = p.W > 8 * p.n_streams;
  if (wide)
    hipLaunchKernelGGL((cap ? mla_combine_kernel<16, true> : mla_combine_kernel<16, false>), grid,
                       dim3(kCombineThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((cap ? mla_combine_kernel<8, true> : mla_combine_kernel<8, false>), grid,
                       dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
