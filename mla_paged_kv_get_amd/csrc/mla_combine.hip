// Combine kernel: merges the splits of each sequence by their lse (FlashMLA
// source walk-through, combine section: each split leaves a partial output and
// lse, and the combine kernel uses lse to fold them into the final result):
//   L = ln sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i,  lse = L.
// Streams with a single split were finished by the decode kernel; streams with
// no tiles (seqlen 0) get o = 0 and lse = -inf.
#include "mla_common.hpp"

namespace mla {

namespace {

constexpr int kCombineRows = 16;  // query rows per workgroup
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(DecodeParams p) {
  const int stream = blockIdx.x;
  const int32_t* split_off = p.meta + meta_split_offset(p.W);
  const int s0 = split_off[stream];
  const int n = split_off[stream + 1] - s0;
  if (n == 1) return;
  const int64_t row_base = (int64_t)stream * p.R_stream;
  const int sub = threadIdx.x >> 7;      // two rows per pass
  const int c = (threadIdx.x & 127) * 4;  // four columns per thread
  for (int rr = sub; rr < kCombineRows; rr += 2) {
    const int row = blockIdx.y * kCombineRows + rr;
    if (row >= p.R_stream) break;
    float mx = -__builtin_huge_valf();
    for (int j = 0; j < n; ++j) mx = fmaxf(mx, p.part_lse[(int64_t)(s0 + j) * p.R_stream + row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = -__builtin_huge_valf();
    if (mx != -__builtin_huge_valf()) {
      float sum = 0.f;
      for (int j = 0; j < n; ++j) sum += __expf(p.part_lse[(int64_t)(s0 + j) * p.R_stream + row] - mx);
      L = mx + __logf(sum);
      for (int j = 0; j < n; ++j) {
        const float lj = p.part_lse[(int64_t)(s0 + j) * p.R_stream + row];
        if (lj == -__builtin_huge_valf()) continue;
        const float wgt = __expf(lj - L);
        const float4 v = *(const float4*)(p.part_o + ((int64_t)(s0 + j) * p.R_stream + row) * kDV + c);
        acc.x += wgt * v.x;
        acc.y += wgt * v.y;
        acc.z += wgt * v.z;
        acc.w += wgt * v.w;
      }
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
