// Device helpers shared by the decode and debug kernels: the LDS layout of a
// 64-token tile and the FP8 -> bf16 decode of the 656-byte token.
#pragma once

#include "mla_common.hpp"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define MLA_LDS __attribute__((address_space(3)))

// LDS tile layout: token t of the page occupies 72 consecutive 16-byte slots
// (t * 72 ...); 16-byte chunk c of its bf16 row is stored at slot
// t * 72 + (c ^ swizzle(t)).  The XOR only touches the low three chunk bits, so
// chunks 0..63 and 64..71 stay in place as groups.  swizzle(t) =
// 4 * bit1(t) + 2 * bit3(t).  On gfx950 a 16-byte LDS read is served 16 lanes
// per clock, the 16 lanes of a clock sharing lane bit 5 and the parity of lane
// bits 2..4 (measured with the LDS bank-conflict counter over a set of access
// patterns); a 64-bit read is served 32 lanes per clock.  With that grouping
// this swizzle keeps both access patterns of the decode kernel free of bank
// conflicts:
//  - the 16x16x32 K operand: lanes 0..15 read 16 consecutive tokens at one
//    chunk, lane groups 16 apart the next chunks, and
//  - the transposed V operand: 4 consecutive tokens (aligned to 4) at 2 adjacent
//    chunks per 16 lanes.
__device__ __forceinline__ int tile_swizzle(int t) { return (((t >> 1) & 1) << 2) | (((t >> 3) & 1) << 1); }
__device__ __forceinline__ int tile_slot(int t, int chunk) { return t * kTokenChunks + (chunk ^ tile_swizzle(t)); }

// Four e4m3fn codes (little-endian bytes of w) times `scale`, each rounded to
// fp32 (RNE) and then to bf16 (RNE); returns the four bf16 packed in two words.
__device__ __forceinline__ u32x2 dequant4(uint32_t w, float scale) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);  // bytes 0, 1 (exact)
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);   // bytes 2, 3
  bf16x2 lo, hi;
  lo.x = (__bf16)(a.x * scale);
  lo.y = (__bf16)(a.y * scale);
  hi.x = (__bf16)(b.x * scale);
  hi.y = (__bf16)(b.y * scale);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// 16 codes (one 16-byte chunk of the FP8 token) -> 16 bf16 in two uint4.
__device__ __forceinline__ void dequant16(u32x4 codes, float scale, u32x4& lo, u32x4& hi) {
  const u32x2 a = dequant4(codes.x, scale), b = dequant4(codes.y, scale);
  const u32x2 c = dequant4(codes.z, scale), d = dequant4(codes.w, scale);
  lo = u32x4{a.x, a.y, b.x, b.y};
  hi = u32x4{c.x, c.y, d.x, d.y};
}

// max(v of lane l, v of lane l ^ 32): v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, so with both
// operands = v each lane ends up holding its own value and its partner's.
// Inline asm because this compiler's builtin for the swap hands back the wrong
// register for one of its two results (checked on gfx950: half the lanes wrong).
__device__ __forceinline__ float halves_max(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// ---- merging decode (the last split of a row tile merges its stream's splits) ----
// A split that knows it is not alone cannot hand its partial result to the
// others through its XCD's L2 (the L2s of the eight XCDs are not coherent with
// each other, and writing back a whole L2 per workgroup is far too slow), so a
// merging call writes partials with device-coherent stores (cache policy sc1:
// written through to memory, as an agent-scope relaxed atomic store is), waits
// for them, then counts itself in with one agent-scope atomic per (stream, row
// tile).  The split that counts last reads every split's partial with
// device-coherent loads, merges them as the combine kernel does and writes o
// and lse; it also resets the counter, so the metadata serves the next call.
constexpr int kCpolSc1 = 16;            // buffer instruction cache policy: sc1
constexpr int kRawBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data, no swizzle

__device__ __forceinline__ void store_coherent_f32(float* ptr, float v) {
  __hip_atomic_store((int*)ptr, __builtin_bit_cast(int, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent_f32(const float* ptr) {
  return __builtin_bit_cast(float, __hip_atomic_load((int*)ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Writes a row tile's partial output (staged in LDS as fp32 rows of `pitch`
// bytes; only rows whose bit is set in `live`, the rest attended nothing) to the
// workspace, counts the split in, and, in the last split of the row tile to
// arrive, merges the stream's nsplit <= kMergeMaxSplits splits (first split id
// s0) into o and lse.  Every thread of the 512-thread workgroup calls it;
// `flag` is one int of LDS.  The split's lse values were written before with
// store_coherent_f32.
template <int kThreadsWG>
__device__ __forceinline__ void merge_split_tile(const DecodeParams& p, MLA_LDS const char* stage, int pitch,
                                                 int stream, int rt, int sid, int s0, int nsplit, int nrows,
                                                 uint64_t live, MLA_LDS int32_t* flag, int tid) {
  constexpr float kNegInf = -__builtin_huge_valf();
  const int64_t R = p.R_stream;
  {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.part_o + ((int64_t)sid * R + rt * kRowTile) * kDV), 0, nrows * kDV * 4, kRawBufferFlags);
#pragma unroll
    for (int k = 0; k < kRowTile * kDV * 4 / 16 / kThreadsWG; ++k) {
      const int c = k * kThreadsWG + tid;
      const int row = c >> 7, off = (c & 127) * 16;
      if (row < nrows && ((live >> row) & 1u))
        __builtin_amdgcn_raw_buffer_store_b128(*(MLA_LDS const u32x4*)(stage + row * pitch + off), rs,
                                               row * kDV * 4 + off, 0, kCpolSc1);
    }
  }
  // every store of this wave (partial rows and lse values) has completed
  // before the barrier, so every store of the workgroup before the count
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int32_t* cnt = p.arrive + (int64_t)stream * p.n_rt + rt;
  if (tid == 0) *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*flag != nsplit - 1) return;  // another split merges
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const __amdgpu_buffer_rsrc_t ps = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.part_o + (int64_t)s0 * R * kDV), 0, (int)(nsplit * R * kDV * 4), kRawBufferFlags);
  const int64_t row_base = (int64_t)stream * R;
  // 64 rows x 64 pieces of 8 columns: four pieces per thread at a time, all
  // their loads in flight together
  constexpr int kBatch = 4;
#pragma unroll 1
  for (int i0 = 0; i0 < kRowTile * (kDV / 8); i0 += kBatch * kThreadsWG) {
    float lj[kBatch][kMergeMaxSplits];
    float4 v[kBatch][kMergeMaxSplits], v2[kBatch][kMergeMaxSplits];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = i0 + t * kThreadsWG + tid;
      const int row = i >> 6, c8 = (i & 63) * 8;
      const int rowj = rt * kRowTile + row;
#pragma unroll
      for (int j = 0; j < kMergeMaxSplits; ++j) {
        const bool ok = j < nsplit && row < nrows;
        const uint32_t off = (uint32_t)(((int64_t)j * R + rowj) * kDV + c8) * 4u;
        lj[t][j] = ok ? load_coherent_f32(p.part_lse + (int64_t)(s0 + j) * R + rowj) : kNegInf;
        v[t][j] = ok ? __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ps, off, 0, kCpolSc1))
                     : make_float4(0.f, 0.f, 0.f, 0.f);
        v2[t][j] = ok ? __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ps, off + 16u, 0, kCpolSc1))
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = i0 + t * kThreadsWG + tid;
      const int row = i >> 6, c8 = (i & 63) * 8;
      if (row >= nrows) continue;
      const int rowj = rt * kRowTile + row;
      float4 acc, acc2;
      const float L = lse_merge<kMergeMaxSplits>(lj[t], v[t], v2[t], acc, acc2);
      *(uint4*)(p.o + (row_base + rowj) * kDV + c8) = pack_bf16x8(acc, acc2);
      if (c8 == 0) p.lse[row_base + rowj] = L;
    }
  }
}

// Merging call, dense cache: streams with no tiles (empty requests) have no
// split to write them, so workgroup g gives streams g, g + grid, ... that are
// empty o = 0 and lse = -inf (the combine kernel does this otherwise).
template <int kThreadsWG>
__device__ __forceinline__ void zero_empty_streams(const DecodeParams& p, int tid) {
  const int32_t* first = p.meta + meta_tile_first(p.W, p.n_streams);
  for (int s = blockIdx.x; s < p.n_streams; s += gridDim.x) {
    if (first[s + 1] != first[s]) continue;
    const int64_t row_base = (int64_t)s * p.R_stream;
    for (int i = tid; i < p.R_stream * (kDV / 8); i += kThreadsWG) {
      const int row = i >> 6, c8 = (i & 63) * 8;
      *(uint4*)(p.o + (row_base + row) * kDV + c8) = make_uint4(0u, 0u, 0u, 0u);
      if (c8 == 0) p.lse[row_base + row] = -__builtin_huge_valf();
    }
  }
}

__device__ __forceinline__ float pick_scale(const u32x4& s, int i) {
  const uint32_t v = i == 0 ? s.x : i == 1 ? s.y : i == 2 ? s.z : s.w;
  return __builtin_bit_cast(float, v);
}

}  // namespace mla
