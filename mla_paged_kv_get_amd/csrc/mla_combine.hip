// Combine kernel: merges the splits of each sequence by their lse (FlashMLA
// source walk-through, combine section: each split leaves a partial output and
// lse, and the combine kernel uses lse to fold them into the final result):
//   L = ln sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i,  lse = L.
// Streams with a single split were finished by the decode kernel; streams with
// no tiles (seqlen 0) get o = 0 and lse = -inf.
//
// One workgroup per (stream, 16 query rows).  Phase 1: one wave per row reduces
// the split lse values (lanes stride over the splits) and stages the split
// weights in LDS.  Phase 2: each thread accumulates four columns of a row over
// the splits, four splits in flight at a time.
#include "mla_common.hpp"

namespace mla {

namespace {

constexpr int kCombineRows = 16;     // query rows per workgroup
constexpr int kCombineThreads = 256;
constexpr int kWeightsLds = 256;     // split weights staged per row

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(DecodeParams p) {
  __shared__ float s_L[kCombineRows];
  __shared__ float s_w[kCombineRows][kWeightsLds];
  const int stream = blockIdx.x;
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int s0 = split_off[stream];
  const int n = split_off[stream + 1] - s0;
  if (n == 1) return;
  const int64_t row_base = (int64_t)stream * p.R_stream;
  const int r0 = blockIdx.y * kCombineRows;
  const int nrows = min(kCombineRows, p.R_stream - r0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr float kNegInf = -__builtin_huge_valf();

  // phase 1: L per row and the first kWeightsLds weights
  for (int rr = wave; rr < nrows; rr += kCombineThreads / 64) {
    const float* lse_col = p.part_lse + (int64_t)s0 * p.R_stream + r0 + rr;
    float mx = kNegInf;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, lse_col[(int64_t)j * p.R_stream]);
    mx = wave_max(mx);
    float sum = 0.f;
    if (mx != kNegInf)
      for (int j = lane; j < n; j += 64) sum += __expf(lse_col[(int64_t)j * p.R_stream] - mx);
    sum = wave_sum(sum);
    const float L = mx == kNegInf ? kNegInf : mx + __logf(sum);
    for (int j = lane; j < min(n, kWeightsLds); j += 64) {
      const float lj = lse_col[(int64_t)j * p.R_stream];
      s_w[rr][j] = (L == kNegInf || lj == kNegInf) ? 0.f : __expf(lj - L);
    }
    if (lane == 0) s_L[rr] = L;
  }
  __syncthreads();

  // phase 2: weighted sum of the split outputs
  const int c = (threadIdx.x & 127) * 4;
  for (int rr = threadIdx.x >> 7; rr < nrows; rr += 2) {
    const int row = r0 + rr;
    const float L = s_L[rr];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* po = p.part_o + ((int64_t)s0 * p.R_stream + row) * kDV + c;
    const int64_t stride = (int64_t)p.R_stream * kDV;
    int j = 0;
    for (; j + 4 <= min(n, kWeightsLds); j += 4) {
      float4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *(const float4*)(po + (j + k) * stride);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = s_w[rr][j + k];
        acc.x += w * v[k].x;
        acc.y += w * v[k].y;
        acc.z += w * v[k].z;
        acc.w += w * v[k].w;
      }
    }
    for (; j < n; ++j) {
      float w;
      if (j < kWeightsLds) {
        w = s_w[rr][j];
      } else {
        const float lj = p.part_lse[(int64_t)(s0 + j) * p.R_stream + row];
        w = (L == kNegInf || lj == kNegInf) ? 0.f : __expf(lj - L);
      }
      if (w == 0.f) continue;
      const float4 v = *(const float4*)(po + j * stride);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 a, b;
    a.x = (__bf16)acc.x;
    a.y = (__bf16)acc.y;
    b.x = (__bf16)acc.z;
    b.y = (__bf16)acc.w;
    *(uint2*)(p.o + (row_base + row) * kDV + c) = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
    if (c == 0) p.lse[row_base + row] = L;
  }
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.n_streams, (p.R_stream + kCombineRows - 1) / kCombineRows);
  hipLaunchKernelGGL(mla_combine_kernel, grid, dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
