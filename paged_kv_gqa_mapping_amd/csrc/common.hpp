// Device helpers shared by the gfx950 kernels: bf16 packing, wave64 DPP
// reductions, the hardware base-2 exponential, and the paged-cache address of
// a token row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
// Online softmax: the running reference max is raised only when a score
// exceeds it by more than kTau (log2 units), so weights stay <= 2^kTau and most
// steps skip the rescale.  Any reference max gives the same quotient o / l.
constexpr float kTau = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// A bf16 value is the high half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// fp32 accumulate of a two-element bf16 dot product: c + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// v_exp_f32: 2^x.  exp2(-inf) = 0, exp2(0) = 1.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Every control used below reads a valid lane for every lane, so bound_ctrl
// never applies; setting it lets the compiler fold the move into the add.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of a
// group gets the same bits (each step adds a pair in both orders, and fp32
// addition commutes).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Combine lane l with lane l ^ 32 through v_permlane32_swap.  With the same
// register as both operands the two results hold, in every lane, the lower-
// and the upper-half value of the pair (lane l < 32: {x[l], x[l+32]}; lane
// l >= 32: {x[l-32], x[l]}), so max and sum below give the same bits in both
// lanes of a pair.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pkv
