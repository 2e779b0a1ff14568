// Instantiations and dispatch of the row-attention kernels (decode split,
// decode reduce, fp32 prefill rows).
#include "row_attn.hpp"

// Compile-time tuning knobs (defaults are the measured choice):
//   PKV_ROW_HPW_MAX  cap on KV heads per wave (8, 4, 2 or 1)
//   PKV_ROW_MAX_ACC  cap on fp32 output accumulators per lane, G * D / (64 / hpw)
//   PKV_ROW_U        tokens per step (0: 4 for bf16 with G <= 4, else 2)
//   PKV_ROW_R        step buffers in the load ring (R - 1 steps in flight; 0: 3 for bf16
//                    decode with G = 4, else 2)
//   PKV_ROW_NT       1: K/V stream loads marked non-temporal (row_attn.hpp)
#ifndef PKV_ROW_HPW_MAX
#define PKV_ROW_HPW_MAX 8
#endif
#ifndef PKV_ROW_MAX_ACC
#define PKV_ROW_MAX_ACC 64
#endif
#ifndef PKV_ROW_U
#define PKV_ROW_U 0
#endif
#ifndef PKV_ROW_R
#define PKV_ROW_R 0
#endif

namespace pkv {

namespace {

// KV heads per wave: the most of {8, 4, 2, 1} that divides num_kv_heads while
// each lane still owns at least one 32-bit word of a row and holds at most 64
// fp32 output accumulators (G heads x D / (64 / hpw) elements); if no choice
// meets the second bound, the smallest that meets the first.
int choose_hpw(int32_t dtype, int32_t head_dim, int32_t num_q_heads, int32_t num_kv_heads) {
  const int elt = dtype == kBF16 ? 2 : 4;
  const int G = num_q_heads / num_kv_heads;
  int fallback = 0;
  for (int hpw : {8, 4, 2, 1}) {
    if (hpw > PKV_ROW_HPW_MAX || num_kv_heads % hpw) continue;
    const int dpl = head_dim / (64 / hpw);
    if (dpl * elt < 4) continue;
    fallback = hpw;
    if (G * dpl <= PKV_ROW_MAX_ACC) return hpw;
  }
  return fallback;
}

template <bool BF16, int D, int HPW, int G, bool PREFILL>
hipError_t launch_one(const RowAttnArgs& a, hipStream_t stream) {
  constexpr int U = PKV_ROW_U ? PKV_ROW_U : ((BF16 && G <= 4) ? 4 : 2);  // tokens per step
  // load ring depth: with non-temporal K/V loads a 3-deep ring (two steps in
  // flight, one wave per SIMD) is 1-6 % faster for G = 4 and neutral for G = 2
  // (G = 8 would need 166 accumulation registers on top of 256 VGPRs)
  constexpr int R = PKV_ROW_R ? PKV_ROW_R : ((BF16 && G == 4 && !PREFILL) ? 3 : 2);
  const int n_hg = a.num_kv_heads / HPW;
  const int64_t rows = PREFILL ? (int64_t)a.max_rows : (int64_t)a.num_splits;
  const int64_t blocks =
      (!PREFILL && a.balance_pieces > 0) ? (int64_t)n_hg * a.balance_pieces : (int64_t)n_hg * a.num_seqs * rows;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (!PREFILL && a.k_new)
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, HPW, G, U, R, PREFILL, !PREFILL>), dim3((unsigned)blocks),
                       dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, HPW, G, U, R, PREFILL, false>), dim3((unsigned)blocks),
                       dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, int D, int HPW, bool PREFILL>
hipError_t by_group(const RowAttnArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_one<BF16, D, HPW, 1, PREFILL>(a, stream);
    case 2: return launch_one<BF16, D, HPW, 2, PREFILL>(a, stream);
    case 4: return launch_one<BF16, D, HPW, 4, PREFILL>(a, stream);
    case 8: return launch_one<BF16, D, HPW, 8, PREFILL>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <bool BF16, int D, bool PREFILL>
hipError_t by_hpw(const RowAttnArgs& a, int hpw, int G, hipStream_t stream) {
  switch (hpw) {
    case 8: return by_group<BF16, D, 8, PREFILL>(a, G, stream);
    case 4: return by_group<BF16, D, 4, PREFILL>(a, G, stream);
    case 2: return by_group<BF16, D, 2, PREFILL>(a, G, stream);
    case 1:
      if constexpr (D * (BF16 ? 2 : 4) / 64 >= 4) return by_group<BF16, D, 1, PREFILL>(a, G, stream);
      break;
  }
  return hipErrorInvalidValue;
}

template <bool PREFILL>
hipError_t dispatch(const RowAttnArgs& a, int32_t dtype, int32_t head_dim, hipStream_t stream) {
  const int hpw = choose_hpw(dtype, head_dim, a.num_q_heads, a.num_kv_heads);
  const int G = a.num_q_heads / a.num_kv_heads;
  if (dtype == kBF16) {
    if (head_dim == 128) return by_hpw<true, 128, PREFILL>(a, hpw, G, stream);
    if (head_dim == 64) return by_hpw<true, 64, PREFILL>(a, hpw, G, stream);
  } else {
    if (head_dim == 128) return by_hpw<false, 128, PREFILL>(a, hpw, G, stream);
    if (head_dim == 64) return by_hpw<false, 64, PREFILL>(a, hpw, G, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool row_attn_supported(int32_t dtype, int32_t head_dim, int32_t num_q_heads, int32_t num_kv_heads) {
  if (dtype != kBF16 && dtype != kF32) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  if (num_kv_heads < 1 || num_q_heads % num_kv_heads) return false;
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  return choose_hpw(dtype, head_dim, num_q_heads, num_kv_heads) != 0;
}

hipError_t launch_row_attn(const RowAttnArgs& a, int32_t dtype, int32_t head_dim, bool prefill, hipStream_t stream) {
  return prefill ? dispatch<true>(a, dtype, head_dim, stream) : dispatch<false>(a, dtype, head_dim, stream);
}

// Pair count up to which the merge gives each (sequence, head) a workgroup.
constexpr int64_t kReduceWidePairs = 1024;

template <bool BF16, int D>
void launch_reduce(const RowAttnArgs& a, bool wide, dim3 grid, dim3 block, hipStream_t stream) {
  if (wide)
    hipLaunchKernelGGL((decode_reduce_kernel<BF16, D, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<BF16, D, false>), grid, block, 0, stream, a);
}

hipError_t launch_decode_reduce(const RowAttnArgs& a, int32_t dtype, int32_t head_dim, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.num_seqs * a.num_q_heads;
  if (pairs <= 0) return hipSuccess;
  if (pairs > 0x7fffffff) return hipErrorInvalidValue;
  // few pairs: a workgroup each, its waves sharing the pair's states; else a
  // wave each (kReduceWaves pairs per workgroup)
  const bool wide = pairs <= kReduceWidePairs;
  dim3 grid((unsigned)(wide ? pairs : (pairs + kReduceWaves - 1) / kReduceWaves)), block(kReduceWaves * 64);
  if (dtype == kBF16 && head_dim == 128) launch_reduce<true, 128>(a, wide, grid, block, stream);
  else if (dtype == kBF16 && head_dim == 64) launch_reduce<true, 64>(a, wide, grid, block, stream);
  else if (dtype == kF32 && head_dim == 128) launch_reduce<false, 128>(a, wide, grid, block, stream);
  else if (dtype == kF32 && head_dim == 64) launch_reduce<false, 64>(a, wide, grid, block, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
