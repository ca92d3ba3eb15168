// Set-up of a sparse prefill call: the prefill reads one contiguous latent KV
// sequence, which the decode path sees as a single request whose pages are
// the sequence's consecutive 64-token pieces.  This kernel writes that
// request's length and its identity page table into the call's workspace, so
// the scheduler and the decode kernel run unchanged on it.
#include "mla_common.hpp"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void mla_prefill_setup_kernel(int32_t* __restrict__ seqlen,
                                                                int32_t* __restrict__ pages, int n_pages, int s_kv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_pages) pages[i] = i;
  if (i == 0) seqlen[0] = s_kv;
}

}  // namespace

hipError_t launch_prefill_setup(int32_t* seqlen, int32_t* pages, int n_pages, int s_kv, hipStream_t stream) {
  const int blocks = (n_pages + 255) / 256;
  hipLaunchKernelGGL(mla_prefill_setup_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, seqlen, pages,
                     n_pages, s_kv);
  return hipGetLastError();
}

}  // namespace mla
