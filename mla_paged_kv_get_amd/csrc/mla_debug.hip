// Test hook: exports the FP8 -> bf16 decode the decode kernel applies when it
// stages a 656-byte token into LDS (same device function), so the decode can be
// checked bit for bit.  One thread per 16-byte chunk of the output row.
#include "mla_device.hpp"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void mla_debug_dequant_kernel(const uint8_t* __restrict__ tokens, int64_t n,
                                                                 uint16_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tok = gid / kTokenChunks;
  const int chunk = (int)(gid % kTokenChunks);  // 16-byte chunk of the 576-dim bf16 row
  if (tok >= n) return;
  const uint8_t* src = tokens + tok * kFp8TokenBytes;
  u32x4* dst = (u32x4*)(out + tok * kDQK) + chunk;
  if (chunk < 64) {
    const int c = chunk >> 1;  // 16-code chunk
    const u32x4 codes = *(const u32x4*)(src + 16 * c);
    const u32x4 sc = *(const u32x4*)(src + kFp8Dims);
    u32x4 lo, hi;
    dequant16(codes, pick_scale(sc, c >> 3), lo, hi);
    *dst = (chunk & 1) ? hi : lo;
  } else {
    *dst = *(const u32x4*)(src + kFp8Dims + 16 + 16 * (chunk - 64));
  }
}

}  // namespace

hipError_t launch_debug_dequant(const uint8_t* tokens, int64_t n, uint16_t* out, hipStream_t stream) {
  const int64_t total = n * kTokenChunks;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(mla_debug_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, tokens, n, out);
  return hipGetLastError();
}

}  // namespace mla
