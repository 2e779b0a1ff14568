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
//
// SHARED mode is the group pass of shared-prefix ("cascade") decode: the
// columns are the decode queries of the members of one group (sequences
// whose first keys are the same cached blocks), the keys one chunk of that
// shared prefix, with no causal mask (every member's token comes after the
// prefix), and the result is each column's unnormalised softmax state (m, l,
// o) written to the member's decode workspace, merged later with the states
// of its own keys.  The shared keys are thus read once per group instead of
// once per member.
#include "common.hpp"
#include "kernels.hpp"

// Column blocks of 32 (position, head) columns per wave (1 or 2); 2 reuses
// every LDS operand fragment twice at one wave per SIMD.
#ifndef PKV_PF_NBW
#define PKV_PF_NBW 1
#endif

// Tiles of K/V whose global loads are in flight while a tile is computed (1 or
// 2 register stages).
#ifndef PKV_PF_DEPTH
#define PKV_PF_DEPTH 2
#endif

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

// UT: every 64-key tile lies in one block (block_size >= 64, or packed K/V), so
// a tile's base address is the same for the whole wave and only the row within
// the tile is per lane.
template <int D, int HW, int NBW, bool SHARED, bool UT>
__global__ __launch_bounds__(256, NBW == 1 ? 2 : 1) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int PB = 4 / HW;           // position blocks (of 32 * NBW) per workgroup
  constexpr int WP = 32 * NBW;         // positions per wave
  constexpr int QP = WP * PB;          // positions per workgroup
  constexpr int KSTEPS = D / 16;       // contraction steps of Q K^T
  constexpr int MD = D / 32;           // 32-row blocks of O^T
  constexpr int KS = D + 8;            // LDS K row stride (elements): 16-byte pad
  constexpr int VS = kKT + 8;          // LDS V^T row stride (elements)
  constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
  constexpr int CPT = CPR / 4;         // K chunks per thread (4 threads per K row)
  constexpr int VT = (kKT / 4) * CPR;  // threads that load V (4 keys x 8 dims each)
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][D * VS];

  const int tid = threadIdx.x;
  // wave-uniform (scalar): the tile loop bounds and the block-id lookups derive from it
  const int wave = uniform(tid >> 6);
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
  // Prefill: sequence b, its query tile `tile` (Lq queries, Lk keys, packed
  // rows from k0).  Shared: group member tile `tile` (Lq members), keys
  // [key_base, key_base + Lk) of the prefix, table row of the group's first
  // member b.
  int b, tile, q0 = 0, Lq, k0 = 0, Lk, key_base = 0, member0 = 0, chunk = 0;
  if constexpr (SHARED) {
    tile = id % a.member_tiles;
    id /= a.member_tiles;
    chunk = id % a.num_chunks;
    const int gi = id / a.num_chunks;
    member0 = a.group_offsets[gi];
    Lq = a.group_offsets[gi + 1] - member0;
    if (tile * QP >= Lq) return;
    b = a.group_seqs[member0];
    const int shared = a.shared_lens[b];
    key_base = chunk * a.chunk_tokens;
    if (key_base >= shared) return;
    Lk = min(shared - key_base, a.chunk_tokens);
  } else {
    b = id % a.num_seqs;
    const int tile_rev = id / a.num_seqs;
    q0 = a.cu_seqlens_q[b];
    Lq = a.cu_seqlens_q[b + 1] - q0;
    k0 = a.cu_seqlens_k[b];
    Lk = a.cu_seqlens_k[b + 1] - k0;
    const int n_qt = (Lq + QP - 1) / QP;
    tile = n_qt - 1 - tile_rev;  // tiles with the most keys are dispatched first
    if (tile < 0) return;
  }

  const int hl = wave % HW;
  const int pb = wave / HW;
  const int h = hg * HW + hl;
  const int g = (hg * HW) / G;
  // Positions are relative to key_base.  Prefill: query i sits at shift + i.
  // Shared: every column sees the whole chunk, as a query at its last key.
  const int shift = Lk - Lq;
  const int w_first = tile * QP + pb * WP;
  const int w_last = min(w_first + WP, Lq) - 1;
  const bool wave_active = w_first < Lq;
  const int w_min_pos = SHARED ? Lk - 1 : shift + w_first;
  const int w_max_pos = SHARED ? Lk - 1 : shift + w_last;
  // column block nb of the wave holds queries (members) w_first + 32 nb + col
  int pos[NBW];
  bool col_valid[NBW];
  int64_t q_row[NBW];  // row of q[., Hq, D] (times Hq, plus the head)
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int qi = w_first + 32 * nb + col;
    col_valid[nb] = qi < Lq;
    pos[nb] = (col_valid[nb] && !SHARED) ? shift + qi : Lk - 1;
    if constexpr (SHARED) {
      q_row[nb] = col_valid[nb] ? (int64_t)a.group_seqs[member0 + qi] * Hq + h : 0;
    } else {
      q_row[nb] = (int64_t)(q0 + qi) * Hq + h;
    }
  }
  const int wg_max_pos = SHARED ? Lk - 1 : shift + min(tile * QP + QP, Lq) - 1;
  const int n_kt = wg_max_pos / kKT + 1;

  // Q^T as the B operand: lane (col, half) holds Q[col][16 kk + 8 half .. +8].
  bf16x8_t qf[NBW][KSTEPS];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const uint16_t* qp = (const uint16_t*)a.q + q_row[nb] * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (col_valid[nb]) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[nb][kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // Tile loads.  K: thread t owns row (t % 16) + 16 (t / 64) and chunks
  // ((t / 16) % 4) + 4 i, so 16 consecutive lanes write one chunk of 16
  // consecutive rows (the row stride keeps them on distinct banks) and each
  // global load instruction reads 64 contiguous bytes of 16 rows.  V: thread t
  // owns keys 4 (t % 16) .. +3 and dims 8 (t / 16) .. +7, so 16 consecutive
  // lanes write the 16 eight-byte key slots of one V^T row (128 contiguous
  // bytes).
  const int32_t* table = a.block_tables ? a.block_tables + (int64_t)b * a.max_blocks_per_seq : nullptr;
  const int lbs = a.log2_block_size;
  const int bs_mask = (1 << lbs) - 1;
  const uint16_t* kbase = (const uint16_t*)a.k;
  const uint16_t* vbase = (const uint16_t*)a.v;
  const int k_row = (tid & 15) + 16 * (tid >> 6);
  const int k_c0 = (tid >> 4) & 3;
  const bool v_loader = wave < VT / 64;  // whole waves (VT is a multiple of 64)
  const int v_kg = tid & 15;
  const int v_dc = tid >> 4;

  // Keys past the end of the sequence (the tail of the last tile) re-read the
  // last key's row: their scores are masked (key > every position) and their
  // weights are exactly 0, so finite data suffices and no zero fill is needed.
  const int last_key = Lk - 1;
  // block id holding key t (relative to key_base; packed K/V: unused)
  auto block_id = [&](int t) -> int32_t { return table ? table[(key_base + min(t, last_key)) >> lbs] : 0; };
  // UT: block id of the tile starting at key t (t <= last_key), the same for every lane
  auto tile_block = [&](int t) -> int32_t { return table ? table[uniform((key_base + t) >> lbs)] : 0; };
  // element offset of key tc's row (tc <= last_key) for KV head g; blk is the block holding tc
  const int row_stride = Hkv * D;
  const int64_t blk_stride = (int64_t)row_stride << lbs;
  const int head_off = g * D;
  auto row_elem = [&](int tc, int32_t blk) -> int64_t {
    if (table) return (int64_t)blk * blk_stride + (((key_base + tc) & bs_mask) * row_stride + head_off);
    return (int64_t)(k0 + tc) * row_stride + head_off;
  };

  static_assert(CPT == 2 || CPT == 4, "head_dim 64 or 128");
  // Prefetched rows of one tile (a stage): K chunks k_c0 + 4 i (i < CPT) and
  // the V rows of keys 4 kg .. 4 kg + 3, passed as separate values so that
  // they stay in registers.
#define PKV_STAGE_PARAMS uint4 &k0r, uint4 &k1r, uint4 &k2r, uint4 &k3r, uint4 &v0, uint4 &v1, uint4 &v2, uint4 &v3
  auto issue_loads = [&](PKV_STAGE_PARAMS, int kt, int32_t bk, int32_t bv) {
    if constexpr (UT) {
      // bk is the tile's block; rows past the end re-read the last key's row
      const int t0 = kt * kKT;
      const int64_t tile = table ? (int64_t)bk * blk_stride + (int64_t)((key_base + t0) & bs_mask) * row_stride
                                 : (int64_t)(k0 + t0) * row_stride;
      const int last = last_key - t0;
      const uint16_t* kp = kbase + tile + (min(k_row, last) * row_stride + head_off + k_c0 * 8);
      k0r = *reinterpret_cast<const uint4*>(kp);
      k1r = *reinterpret_cast<const uint4*>(kp + 32);
      if constexpr (CPT == 4) {
        k2r = *reinterpret_cast<const uint4*>(kp + 64);
        k3r = *reinterpret_cast<const uint4*>(kp + 96);
      }
      if (v_loader) {
        const uint16_t* vp = vbase + tile + (head_off + v_dc * 8);
        const int tv = 4 * v_kg;
        v0 = *reinterpret_cast<const uint4*>(vp + min(tv, last) * row_stride);
        v1 = *reinterpret_cast<const uint4*>(vp + min(tv + 1, last) * row_stride);
        v2 = *reinterpret_cast<const uint4*>(vp + min(tv + 2, last) * row_stride);
        v3 = *reinterpret_cast<const uint4*>(vp + min(tv + 3, last) * row_stride);
      }
      return;
    }
    const int64_t ek = row_elem(min(kt * kKT + k_row, last_key), bk) + k_c0 * 8;
    k0r = *reinterpret_cast<const uint4*>(kbase + ek);
    k1r = *reinterpret_cast<const uint4*>(kbase + ek + 32);
    if constexpr (CPT == 4) {
      k2r = *reinterpret_cast<const uint4*>(kbase + ek + 64);
      k3r = *reinterpret_cast<const uint4*>(kbase + ek + 96);
    }
    if (v_loader) {
      // the 4 keys are consecutive rows of one block (4-aligned, block_size >= 8);
      // keys past the end all read the last key's row
      const int tv = kt * kKT + 4 * v_kg;
      const int tvc = min(tv, last_key);
      const int64_t ev = row_elem(tvc, bv) + v_dc * 8;
      auto row = [&](int i) {
        return *reinterpret_cast<const uint4*>(vbase + ev + (int64_t)((min(tv + i, last_key) - tvc) * row_stride));
      };
      v0 = row(0);
      v1 = row(1);
      v2 = row(2);
      v3 = row(3);
    }
  };
  auto write_lds = [&](PKV_STAGE_PARAMS, int buf) {
    uint16_t* kd = &lds_k[buf][k_row * KS + k_c0 * 8];
    *reinterpret_cast<uint4*>(kd) = k0r;
    *reinterpret_cast<uint4*>(kd + 32) = k1r;
    if constexpr (CPT == 4) {
      *reinterpret_cast<uint4*>(kd + 64) = k2r;
      *reinterpret_cast<uint4*>(kd + 96) = k3r;
    }
    if (v_loader) {
      const int vc = vt_column(4 * v_kg);
      const uint32_t r0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t r1[4] = {v1.x, v1.y, v1.z, v1.w};
      const uint32_t r2[4] = {v2.x, v2.y, v2.z, v2.w};
      const uint32_t r3[4] = {v3.x, v3.y, v3.z, v3.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = v_dc * 8 + 2 * w;
        // v_perm_b32: selector bytes 0-3 pick from the second operand, 4-7 from the first
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);  // (key 0, key 1) of dim d
        lo.y = __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u);  // (key 2, key 3)
        hi.x = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);  // dim d + 1
        hi.y = __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u);
        *reinterpret_cast<uint2*>(&lds_v[buf][d * VS + vc]) = lo;
        *reinterpret_cast<uint2*>(&lds_v[buf][(d + 1) * VS + vc]) = hi;
      }
    }
  };

  f32x16_t acc_o[NBW][MD];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[nb][md][r] = 0.f;
  float m[NBW], lsum[NBW];  // running reference max (log2 units) and this half-wave's weight sum, per column
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    m[nb] = kNegInf;
    lsum[nb] = 0.f;
  }
  const float c = a.scale_log2;  // > 0
  const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

  auto compute = [&](int buf, int key0) {
    // S^T = K Q^T (raw scores); each K fragment feeds the NBW column blocks
    f32x16_t acc_s[NBW][2];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[nb][mb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t af = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&lds_k[buf][(mb * 32 + col) * KS + 16 * kk + 8 * half]));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          acc_s[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[nb][kk], acc_s[nb][mb], 0, 0, 0);
      }
    }
    uint32_t pw[NBW][16];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      // causal mask (only on tiles that reach past the block's first position):
      // key key0 + off(r) with off(r) = mb*32 + (r/4)*8 + half*4 + r%4 is
      // visible iff off(r) - half*4 <= pos - key0 - half*4
      if (key0 + kKT - 1 > w_min_pos + (SHARED ? 0 : 32 * nb)) {
        const int lim = pos[nb] - key0 - half * 4;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb * 32 + (r >> 2) * 8 + (r & 3) > lim) acc_s[nb][mb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[nb][mb][r]);
      mx = halves_max(mx) * c;  // c > 0, so the max commutes with the scaling
      if (wave_any(mx > m[nb] + kTau)) {
        const float mn = fmaxf(m[nb], mx);
        const float alpha = exp2_hw(m[nb] - mn);
        m[nb] = mn;
        lsum[nb] *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[nb][md][r] *= alpha;
      }
      // P^T = 2^(c s - m), rounded to bf16, as the B operand of the four 16-key steps
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float s0 = acc_s[nb][i >> 3][(2 * i) & 15];
        const float s1 = acc_s[nb][i >> 3][(2 * i + 1) & 15];
        pw[nb][i] = pack_bf16x2(exp2_hw(fmaf(s0, c, -m[nb])), exp2_hw(fmaf(s1, c, -m[nb])));
        lsum[nb] = dot2_bf16(pw[nb][i], kOnes, lsum[nb]);
      }
    }
    // O^T += V^T P^T; each V^T fragment feeds the NBW column blocks
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const bf16x8_t af = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&lds_v[buf][(md * 32 + col) * VS + 16 * ks + 8 * half]));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const bf16x8_t bf = __builtin_bit_cast(
              bf16x8_t, make_uint4(pw[nb][4 * ks], pw[nb][4 * ks + 1], pw[nb][4 * ks + 2], pw[nb][4 * ks + 3]));
          acc_o[nb][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc_o[nb][md], 0, 0, 0);
        }
      }
    }
  };

  const int n_kt_wave = wave_active ? min(n_kt, w_max_pos / kKT + 1) : 0;
  // block ids of the next tile to load (run one tile ahead of its loads)
  int32_t bk, bv = 0;
  auto next_ids = [&](int t) {
    if constexpr (UT) {
      bk = tile_block(t * kKT);
    } else {
      bk = block_id(t * kKT + k_row);
      bv = block_id(t * kKT + 4 * v_kg);
    }
  };
  next_ids(0);
#if PKV_PF_DEPTH == 2
  // Pipeline: while tile kt is computed from LDS, the global loads of tiles
  // kt+1 and kt+2 are in flight in two register stages (tile t in stage t % 2),
  // so a load has two tiles' compute time to arrive.  One barrier per tile.
  // The tiles past this wave's last position are only loaded for the other
  // waves (the last loop), which keeps the compute loop free of a
  // data-dependent skip.
  uint4 a0, a1, a2, a3, a4, a5, a6, a7;  // stage 0
  uint4 b0, b1, b2, b3, b4, b5, b6, b7;  // stage 1
#define PKV_S0 a0, a1, a2, a3, a4, a5, a6, a7
#define PKV_S1 b0, b1, b2, b3, b4, b5, b6, b7
  issue_loads(PKV_S0, 0, bk, bv);
  if (n_kt > 1) {
    next_ids(1);
    issue_loads(PKV_S1, 1, bk, bv);
    if (n_kt > 2) next_ids(2);
  }
  write_lds(PKV_S0, 0);
  __syncthreads();
  if (n_kt > 2) {
    const int32_t ck = bk, cv = bv;
    if (n_kt > 3) next_ids(3);
    issue_loads(PKV_S0, 2, ck, cv);
  }
  // tile kt: compute it, move tile kt+1 from its stage `wr` to LDS, refill `wr` with tile kt+3
  auto step = [&](int kt, PKV_STAGE_PARAMS, bool with_compute) {
    if (with_compute) compute(kt & 1, kt * kKT);
    if (kt + 1 < n_kt) write_lds(k0r, k1r, k2r, k3r, v0, v1, v2, v3, (kt & 1) ^ 1);
    if (kt + 3 < n_kt) {
      // the next tile's block ids are requested before this tile's rows, so that
      // waiting for them later never waits for these rows (loads retire in order)
      const int32_t ck = bk, cv = bv;
      if (kt + 4 < n_kt) next_ids(kt + 4);
      issue_loads(k0r, k1r, k2r, k3r, v0, v1, v2, v3, kt + 3, ck, cv);
    }
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 1 < n_kt_wave; kt += 2) {
    step(kt, PKV_S1, true);
    step(kt + 1, PKV_S0, true);
  }
  if (kt < n_kt_wave) step(kt++, PKV_S1, true);
  for (; kt < n_kt; ++kt) {
    if (kt & 1)
      step(kt, PKV_S0, false);
    else
      step(kt, PKV_S1, false);
  }
#undef PKV_S0
#undef PKV_S1
#else
  // Pipeline: tile kt+1's global loads are in flight while tile kt is computed
  // from LDS; block ids run two tiles ahead.  One barrier per tile.
  uint4 a0, a1, a2, a3, a4, a5, a6, a7;
#define PKV_S0 a0, a1, a2, a3, a4, a5, a6, a7
  issue_loads(PKV_S0, 0, bk, bv);
  if (n_kt > 1) next_ids(1);
  write_lds(PKV_S0, 0);
  __syncthreads();
  auto advance = [&](int kt) {
    if (kt + 1 < n_kt) {
      issue_loads(PKV_S0, kt + 1, bk, bv);
      if (kt + 2 < n_kt) next_ids(kt + 2);
    }
  };
  int kt = 0;
  for (; kt < n_kt_wave; ++kt) {
    advance(kt);
    compute(kt & 1, kt * kKT);
    if (kt + 1 < n_kt) write_lds(PKV_S0, (kt & 1) ^ 1);
    __syncthreads();
  }
  for (; kt < n_kt; ++kt) {
    advance(kt);
    if (kt + 1 < n_kt) write_lds(PKV_S0, (kt & 1) ^ 1);
    __syncthreads();
  }
#undef PKV_S0
#endif
#undef PKV_STAGE_PARAMS

  if (!wave_active) return;
  if constexpr (SHARED) {
    // unnormalised state of each column at slot slot0 + chunk of its member's pair
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const float l = halves_sum(lsum[nb]);
      if (!col_valid[nb]) continue;
      const int64_t slot = q_row[nb] * a.ws_stride + a.slot0 + chunk;
      float* wo = a.ws_o + slot * D + half * 4;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = rr * 4;
          *reinterpret_cast<float4*>(wo + md * 32 + rr * 8) =
              make_float4(acc_o[nb][md][r], acc_o[nb][md][r + 1], acc_o[nb][md][r + 2], acc_o[nb][md][r + 3]);
        }
      if (half == 0) {
        a.ws_ml[slot * 2] = m[nb];
        a.ws_ml[slot * 2 + 1] = l;
      }
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (!col_valid[nb]) continue;
    const float inv = 1.0f / halves_sum(lsum[nb]);
    uint16_t* op = (uint16_t*)a.out + q_row[nb] * D + half * 4;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rr * 4;
        uint2 w;
        w.x = pack_bf16x2(acc_o[nb][md][r] * inv, acc_o[nb][md][r + 1] * inv);
        w.y = pack_bf16x2(acc_o[nb][md][r + 2] * inv, acc_o[nb][md][r + 3] * inv);
        *reinterpret_cast<uint2*>(op + md * 32 + rr * 8) = w;
      }
    }
  }
}

}  // namespace

namespace {

int heads_per_wave(int32_t num_q_heads, int32_t num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

template <bool SHARED>
hipError_t launch(const PrefillArgs& a, int32_t head_dim, int64_t blocks, int HW, hipStream_t stream) {
  constexpr int NBW = PKV_PF_NBW;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(256);
  const bool ut = !a.block_tables || a.log2_block_size >= 6;  // a 64-key tile never crosses a block
#define PKV_PREFILL_CASE(DD, HH)                                                                      \
  if (head_dim == DD && HW == HH) {                                                                   \
    if (ut)                                                                                           \
      hipLaunchKernelGGL((prefill_mfma_kernel<DD, HH, NBW, SHARED, true>), grid, block, 0, stream, a);  \
    else                                                                                              \
      hipLaunchKernelGGL((prefill_mfma_kernel<DD, HH, NBW, SHARED, false>), grid, block, 0, stream, a); \
    return hipGetLastError();                                                                         \
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

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int HW = heads_per_wave(a.num_q_heads, a.num_kv_heads);
  const int QP = 32 * PKV_PF_NBW * (4 / HW);
  const int64_t n_qt = (a.max_seqlen_q + QP - 1) / QP;
  return launch<false>(a, head_dim, n_qt * a.num_seqs * (a.num_q_heads / HW), HW, stream);
}

int shared_prefix_members_per_wg(int32_t num_q_heads, int32_t num_kv_heads) {
  return 32 * PKV_PF_NBW * (4 / heads_per_wave(num_q_heads, num_kv_heads));
}

int64_t shared_prefix_wgs_per_chunk(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_groups,
                                    int32_t max_group_size) {
  const int per_wg = shared_prefix_members_per_wg(num_q_heads, num_kv_heads);
  const int64_t tiles = ((max_group_size > 1 ? max_group_size : 1) + per_wg - 1) / per_wg;
  return (int64_t)num_groups * tiles * (num_q_heads / heads_per_wave(num_q_heads, num_kv_heads));
}

hipError_t launch_shared_prefix_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int HW = heads_per_wave(a.num_q_heads, a.num_kv_heads);
  const int64_t blocks = (int64_t)a.num_groups * a.num_chunks * a.member_tiles * (a.num_q_heads / HW);
  return launch<true>(a, head_dim, blocks, HW, stream);
}

}  // namespace pkv
