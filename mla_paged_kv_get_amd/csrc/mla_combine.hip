// Combine kernel: merges the splits of each sequence by their lse (FlashMLA
// source walk-through, combine section: each split leaves a partial output and
// lse, and the combine kernel uses lse to fold them into the final result):
//   L = ln sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i,  lse = L.
// Streams with a single split were finished by the decode kernel; streams with
// no tiles (seqlen 0) get o = 0 and lse = -inf.
//
// One thread per (query row, 8 columns): it reads the row's split lse values
// (the same addresses for all 64 threads of a row, so one request per wave),
// forms L and the weights itself, and issues its split outputs' loads eight
// at a time, so a workgroup pays one memory round trip per eight splits instead
// of one per row it visits.  With at most sixteen splits the lse values and
// the split outputs are loaded together: one round trip in all.
#include "mla_common.hpp"

namespace mla {

namespace {

constexpr int kCombineThreads = 256;  // four rows x 64 threads (8 columns each)
constexpr int kCombineBatch = 8;  // split outputs in flight per thread

// kCombineFused: up to this many splits, the lse values and the outputs are
// loaded together (8 or 16; the wider variant holds more VGPRs, so fewer waves
// fit on a CU, and the host uses it only when streams have many splits).
template <int kCombineFused>
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(DecodeParams p) {
  const int stream = blockIdx.x;
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int s0 = split_off[stream];
  const int n = split_off[stream + 1] - s0;
  if (n == 1) return;  // finished by the decode kernel
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= p.R_stream) return;
  const int c = (threadIdx.x & 63) * 8;
  const int64_t row_base = (int64_t)stream * p.R_stream;
  constexpr float kNegInf = -__builtin_huge_valf();
  const float* lse_col = p.part_lse + (int64_t)s0 * p.R_stream + row;  // split j at j * R_stream
  const float* po = p.part_o + ((int64_t)s0 * p.R_stream + row) * kDV + c;
  const int64_t stride = (int64_t)p.R_stream * kDV;

  auto write_out = [&](const float4& acc, const float4& acc2, float L) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 a, b, d, e;
    a.x = (__bf16)acc.x;
    a.y = (__bf16)acc.y;
    b.x = (__bf16)acc.z;
    b.y = (__bf16)acc.w;
    d.x = (__bf16)acc2.x;
    d.y = (__bf16)acc2.y;
    e.x = (__bf16)acc2.z;
    e.y = (__bf16)acc2.w;
    *(uint4*)(p.o + (row_base + row) * kDV + c) =
        make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, d),
                   __builtin_bit_cast(uint32_t, e));
    if (c == 0) p.lse[row_base + row] = L;
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acc2 = acc;

  if (n <= kCombineFused) {
    // Every split's output is loaded together with the lse values, before its
    // weight is known.  L = ln sum_j exp(lse_j), evaluated around the largest
    // lse; a split with lse = -inf (empty) has weight 0 and its output is not
    // used.
    float lj[kCombineFused];
    float4 v[kCombineFused], v2[kCombineFused];
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) {
      lj[k] = k < n ? lse_col[(int64_t)k * p.R_stream] : kNegInf;
      v[k] = k < n ? *(const float4*)(po + k * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
      v2[k] = k < n ? *(const float4*)(po + k * stride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx = kNegInf;
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) mx = fmaxf(mx, lj[k]);
    if (mx == kNegInf) {
      write_out(acc, acc2, kNegInf);
      return;
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) sum += lj[k] == kNegInf ? 0.f : __expf(lj[k] - mx);
    const float L = mx + __logf(sum);
#pragma unroll
    for (int k = 0; k < kCombineFused; ++k) {
      if (lj[k] == kNegInf) continue;
      const float w = __expf(lj[k] - L);
      acc.x += w * v[k].x;
      acc.y += w * v[k].y;
      acc.z += w * v[k].z;
      acc.w += w * v[k].w;
      acc2.x += w * v2[k].x;
      acc2.y += w * v2[k].y;
      acc2.z += w * v2[k].z;
      acc2.w += w * v2[k].w;
    }
    write_out(acc, acc2, L);
    return;
  }

  // more splits: L first (the lse values), then the outputs eight at a time
  float mx = kNegInf;
  for (int j = 0; j < n; ++j) mx = fmaxf(mx, lse_col[(int64_t)j * p.R_stream]);
  float sum = 0.f;
  if (mx != kNegInf)
    for (int j = 0; j < n; ++j) sum += __expf(lse_col[(int64_t)j * p.R_stream] - mx);
  const float L = mx == kNegInf ? kNegInf : mx + __logf(sum);
  if (L != kNegInf) {
    for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
      float4 v[kCombineBatch], v2[kCombineBatch];
      float w[kCombineBatch];
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) {
        const int j = j0 + k;
        const float lj = j < n ? lse_col[(int64_t)j * p.R_stream] : kNegInf;
        // an empty split (lse = -inf) carries weight 0 and its output is not read
        w[k] = lj == kNegInf ? 0.f : __expf(lj - L);
        v[k] = w[k] != 0.f ? *(const float4*)(po + j * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
        v2[k] = w[k] != 0.f ? *(const float4*)(po + j * stride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) {
        acc.x += w[k] * v[k].x;
        acc.y += w[k] * v[k].y;
        acc.z += w[k] * v[k].z;
        acc.w += w[k] * v[k].w;
        acc2.x += w[k] * v2[k].x;
        acc2.y += w[k] * v2[k].y;
        acc2.z += w[k] * v2[k].z;
        acc2.w += w[k] * v2[k].w;
      }
    }
  }
  write_out(acc, acc2, L);
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.n_streams, (p.R_stream + 3) / 4);
  // more than 8 workers per stream: streams are likely cut into more than 8 splits
  if (p.W > 8 * p.n_streams)
    hipLaunchKernelGGL(mla_combine_kernel<16>, grid, dim3(kCombineThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(mla_combine_kernel<8>, grid, dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
