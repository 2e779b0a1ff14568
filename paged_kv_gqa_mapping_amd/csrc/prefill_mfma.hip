// Causal varlen prefill attention on the gfx950 matrix cores (bf16 operands,
// fp32 accumulation), over paged or packed K/V.
//
// Work split: a workgroup (4 waves) takes one sequence, one group of HW query
// heads that share a KV head, and QP = 32 * (4 / HW) consecutive query
// positions; each wave owns 32 (position, head) columns.  The workgroup walks
// the key axis in tiles of 64 keys up to its last query's position, staging
// each K tile (row-major) and V tile (transposed) in LDS once for all 4
// waves, i.e. once for the whole GQA head group.
//
// Per tile and wave, with v_mfma_f32_32x32x16_bf16:
//   S^T[key][col] = K_tile * Q^T     (2 key blocks x D/16 steps)
//   online softmax per column: the accumulator gives each lane one column and
//   16 keys per key block, so the row max and sum are in-lane plus one
//   half-wave exchange;
//   O^T[d][col] += V^T * P^T         (D/32 blocks x 4 steps), where P^T is the
//   S^T accumulator itself, rounded to bf16: the lane/register layout of an
//   MFMA result is the layout of its B operand up to a fixed permutation of
//   the 16 keys of each step, and V^T is written to LDS in that permuted key
//   order so no data moves between lanes.
// Query i of a sequence sits at position Lk - Lq + i and sees keys <= it; the
// mask is applied only on tiles that reach past a wave's first position.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kKT = 64;  // keys per tile

// Column of key k (0..63) of a tile inside a V^T row: within each group of 16
// keys, lane half h and slot j of the MFMA B operand hold key (j/4)*8 + h*4 +
// j%4, so key k is stored at h*8 + j.
__device__ __forceinline__ int vt_column(int k) {
  const int k16 = k & 15;
  return (k & ~15) + ((k16 & 7) >> 2) * 8 + (k16 >> 3) * 4 + (k16 & 3);
}

template <int D, int HW>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int PB = 4 / HW;           // 32-position blocks per workgroup
  constexpr int QP = 32 * PB;          // positions per workgroup
  constexpr int KSTEPS = D / 16;       // contraction steps of Q K^T
  constexpr int MD = D / 32;           // 32-row blocks of O^T
  constexpr int KS = D + 8;            // LDS K row stride (elements): 16-byte pad
  constexpr int VS = kKT + 8;          // LDS V^T row stride (elements)
  constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kKT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[D * VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int NHG = Hq / HW;

  int id = blockIdx.x;
  const int hg = id % NHG;
  id /= NHG;
  const int b = id % a.num_seqs;
  const int tile_rev = id / a.num_seqs;
  const int q0 = a.cu_seqlens_q[b];
  const int Lq = a.cu_seqlens_q[b + 1] - q0;
  const int k0 = a.cu_seqlens_k[b];
  const int Lk = a.cu_seqlens_k[b + 1] - k0;
  const int n_qt = (Lq + QP - 1) / QP;
  const int tile = n_qt - 1 - tile_rev;  // tiles with the most keys are dispatched first
  if (tile < 0) return;

  const int hl = wave % HW;
  const int pb = wave / HW;
  const int h = hg * HW + hl;
  const int g = (hg * HW) / G;
  const int shift = Lk - Lq;  // position of query i is shift + i
  const int w_first = tile * QP + pb * 32;
  const int w_last = min(w_first + 32, Lq) - 1;
  const bool wave_active = w_first < Lq;
  const int w_min_pos = shift + w_first;
  const int w_max_pos = shift + w_last;
  const int qi = w_first + col;
  const bool col_valid = qi < Lq;
  const int pos = col_valid ? shift + qi : Lk - 1;
  const int wg_max_pos = shift + min(tile * QP + QP, Lq) - 1;
  const int n_kt = wg_max_pos / kKT + 1;

  // Q^T as the B operand: lane (col, half) holds Q[col][16 kk + 8 half .. +8].
  bf16x8_t qf[KSTEPS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)(q0 + qi) * Hq + h) * D + 8 * half;
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (col_valid) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  const int32_t* table = a.block_tables ? a.block_tables + (int64_t)b * a.max_blocks_per_seq : nullptr;
  const int bs_mask = (1 << a.log2_block_size) - 1;
  const uint16_t* kbase = (const uint16_t*)a.k;
  const uint16_t* vbase = (const uint16_t*)a.v;
  // element offset of key t's row for KV head g
  auto row_elem = [&](int t) -> int64_t {
    int64_t r;
    if (table) {
      const int64_t blk = table[t >> a.log2_block_size];
      r = (blk << a.log2_block_size) + (t & bs_mask);
    } else {
      r = (int64_t)k0 + t;
    }
    return (r * Hkv + g) * D;
  };

  f32x16_t acc_o[MD];
  for (int md = 0; md < MD; ++md)
    for (int r = 0; r < 16; ++r) acc_o[md][r] = 0.f;
  float m = kNegInf;  // running reference max of this lane's column (log2 units)
  float lsum = 0.f;   // this half-wave's share of the column's weight sum
  const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * kKT;
    __syncthreads();
    // K tile, row-major: chunk id -> (row, 16-byte chunk).
    for (int idc = tid; idc < kKT * CPR; idc += 256) {
      const int row = idc / CPR;
      const int ch = idc % CPR;
      const int t = key0 + row;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (t < Lk) x = *reinterpret_cast<const uint4*>(kbase + row_elem(t) + ch * 8);
      *reinterpret_cast<uint4*>(&lds_k[row * KS + ch * 8]) = x;
    }
    // V tile, transposed: 4 keys x 8 dims per thread.
    if (tid < (kKT / 4) * CPR) {
      const int kg = tid / CPR;
      const int dc = tid % CPR;
      uint4 r[4];
      for (int i = 0; i < 4; ++i) {
        const int t = key0 + kg * 4 + i;
        r[i] = make_uint4(0, 0, 0, 0);
        if (t < Lk) r[i] = *reinterpret_cast<const uint4*>(vbase + row_elem(t) + dc * 8);
      }
      const int vc = vt_column(kg * 4);
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
      for (int w = 0; w < 4; ++w) {
        const int d = dc * 8 + 2 * w;
        uint2 lo, hi;
        lo.x = (w0[w] & 0xffffu) | (w1[w] << 16);
        lo.y = (w2[w] & 0xffffu) | (w3[w] << 16);
        hi.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
        hi.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
        *reinterpret_cast<uint2*>(&lds_v[d * VS + vc]) = lo;
        *reinterpret_cast<uint2*>(&lds_v[(d + 1) * VS + vc]) = hi;
      }
    }
    __syncthreads();
    if (!wave_active || key0 > w_max_pos) continue;

    // S^T = K Q^T
    f32x16_t acc_s[2];
    for (int mb = 0; mb < 2; ++mb)
      for (int r = 0; r < 16; ++r) acc_s[mb][r] = 0.f;
    for (int kk = 0; kk < KSTEPS; ++kk) {
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t af =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&lds_k[(mb * 32 + col) * KS + 16 * kk + 8 * half]));
        acc_s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], acc_s[mb], 0, 0, 0);
      }
    }

    // online softmax over this tile's keys for this lane's column
    const bool diag = key0 + kKT - 1 > w_min_pos;
    float s[32];
    float mx = kNegInf;
    for (int mb = 0; mb < 2; ++mb) {
      for (int r = 0; r < 16; ++r) {
        float v = acc_s[mb][r] * a.scale_log2;
        if (diag) {
          const int key = key0 + mb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          if (key > pos) v = kNegInf;
        }
        s[mb * 16 + r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = halves_max(mx);
    if (wave_any(mx > m + kTau)) {
      const float mn = fmaxf(m, mx);
      const float alpha = exp2_hw(m - mn);
      m = mn;
      lsum *= alpha;
      for (int md = 0; md < MD; ++md)
        for (int r = 0; r < 16; ++r) acc_o[md][r] *= alpha;
    }
    uint32_t pw[16];
    for (int i = 0; i < 16; ++i) {
      pw[i] = pack_bf16x2(exp2_hw(s[2 * i] - m), exp2_hw(s[2 * i + 1] - m));
      lsum = dot2_bf16(pw[i], kOnes, lsum);
    }

    // O^T += V^T P^T
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]));
      for (int md = 0; md < MD; ++md) {
        const bf16x8_t af =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&lds_v[(md * 32 + col) * VS + 16 * ks + 8 * half]));
        acc_o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc_o[md], 0, 0, 0);
      }
    }
  }

  if (!wave_active || !col_valid) return;
  const float inv = 1.0f / halves_sum(lsum);
  uint16_t* op = (uint16_t*)a.out + ((int64_t)(q0 + qi) * Hq + h) * D + half * 4;
  for (int md = 0; md < MD; ++md) {
    for (int rr = 0; rr < 4; ++rr) {
      const int r = rr * 4;
      uint2 w;
      w.x = pack_bf16x2(acc_o[md][r] * inv, acc_o[md][r + 1] * inv);
      w.y = pack_bf16x2(acc_o[md][r + 2] * inv, acc_o[md][r + 3] * inv);
      *reinterpret_cast<uint2*>(op + md * 32 + rr * 8) = w;
    }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int QP = 32 * (4 / HW);
  const int64_t n_qt = (a.max_seqlen_q + QP - 1) / QP;
  const int64_t blocks = n_qt * a.num_seqs * (a.num_q_heads / HW);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(256);
#define PKV_PREFILL_CASE(DD, HH)                                                              \
  if (head_dim == DD && HW == HH) {                                                           \
    hipLaunchKernelGGL((prefill_mfma_kernel<DD, HH>), grid, block, 0, stream, a);             \
    return hipGetLastError();                                                                 \
  }
  PKV_PREFILL_CASE(128, 4)
  PKV_PREFILL_CASE(128, 2)
  PKV_PREFILL_CASE(128, 1)
  PKV_PREFILL_CASE(64, 4)
  PKV_PREFILL_CASE(64, 2)
  PKV_PREFILL_CASE(64, 1)
#undef PKV_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
