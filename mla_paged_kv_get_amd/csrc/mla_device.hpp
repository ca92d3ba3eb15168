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

__device__ __forceinline__ float pick_scale(const u32x4& s, int i) {
  const uint32_t v = i == 0 ? s.x : i == 1 ? s.y : i == 2 ? s.z : s.w;
  return __builtin_bit_cast(float, v);
}

}  // namespace mla
