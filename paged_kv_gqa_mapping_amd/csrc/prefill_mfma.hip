// Causal varlen prefill attention on the gfx950 matrix cores (bf16 operands,
// fp32 accumulation), over paged or packed K/V.
//
// Work split: a workgroup (8 waves, two per SIMD) takes one sequence, one group
// of HW query heads that share a KV head, and QP = 32 * (8 / HW) consecutive
// query positions: 8 column blocks of 32 (position, head) columns, wave w
// holding head w % HW and positions 32 * (w / HW) .. +31 of the tile.  The
// workgroup walks the key axis in tiles of 128 keys up to its last query's
// position; each K and V tile is staged in LDS once for the whole GQA head
// group, i.e. for 256 columns.  The query tiles of one (sequence, head group)
// run back to back on one XCD, so that they share the K/V tiles through its L2.
//
// Tile staging: the global -> LDS copies are direct (global_load_lds_dwordx4:
// 64 lanes x 16 bytes per instruction, a wave-uniform base address in SGPRs
// plus a per-lane offset fixed for the whole launch) into tile buffers (two
// for K, three for V), so that one tile is in flight while another is
// computed, with no register staging.  K and V are stored row-major (one row per key, no
// padding); the 16-byte slot that holds chunk c of key row k is rotated by
// the key (K: (c + k) mod D/8; V: (c + 4 (k mod 4)) mod 16 for D = 128, (c + 4
// (k / 2 mod 2)) mod 8 for D = 64), which keeps the fragment reads below free
// of bank conflicts.
//
// Per tile and wave, with v_mfma_f32_32x32x16_bf16:
//   S^T[key][col] = K_tile * Q^T     (4 key blocks x D/16 steps, ds_read_b128)
//   online softmax per column: the accumulator gives each lane one column and
//   16 keys per key block, so the row max and sum are in-lane plus one
//   half-wave exchange;
//   O^T[d][col] += V^T * P^T         (D/32 blocks x 8 steps of 16 keys), where P^T is the
//   S^T accumulator itself, rounded to bf16.  The lane/register layout of an
//   MFMA result is that of its B operand up to a fixed permutation of the 16
//   keys of each step; the V^T fragments are read with ds_read_b64_tr_b16
//   (a transposing LDS read: in each 16-lane group, lane l receives element
//   l % 4 of the 8-byte rows addressed by lanes l / 4 + 4 j, j = 0..3) with
//   row addresses chosen in that permuted key order, so no data moves between
//   lanes.
// Query i of a sequence sits at position Lk - Lq + i and sees keys <= it; the
// mask is applied only on tiles that reach past a column block's first position.
//
// SHARED mode is the group pass of shared-prefix ("cascade") decode: the
// columns are the decode queries of the members of one group (sequences
// whose first keys are the same cached blocks), the keys one chunk of that
// shared prefix, with no causal mask (every member's token comes after the
// prefix), and the result is each column's unnormalised softmax state (m, l,
// o) written to the member's decode workspace, merged later with the states
// of its own keys.  The shared keys are thus read once per group instead of
// once per member.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

// Keys per tile: 128 (4.4 % faster than 64: half the waits, barriers and copy
// issues per key); one tile's copies are in flight while another is
// computed, ahead by a tile's compute time.
constexpr int kKT = 128;
constexpr int kKB = kKT / 32;  // 32-key blocks per tile
constexpr int kCB = 8;    // column blocks per workgroup
// Skewed schedule: waves 4-7 (which share SIMDs with waves 0-3) multiply a
// tile's weights by V one tile later, after the next barrier, so that the two
// waves of a SIMD are in different phases (one on the matrix core, the other
// in the softmax) instead of in the same one.  V then needs a third buffer.
#ifndef PKV_PREFILL_SKEW
#define PKV_PREFILL_SKEW 1
#endif
constexpr bool kSkew = PKV_PREFILL_SKEW != 0;
// Compile-time tuning knobs (defaults are the measured choice): LDS fragment
// reads in flight ahead of the MFMAs (K, V^T), and the wave priority taken
// while a wave issues its matrix products (0: never raised).
#ifndef PKV_PREFILL_KPF
#define PKV_PREFILL_KPF 4
#endif
#ifndef PKV_PREFILL_VPF
#define PKV_PREFILL_VPF 3
#endif
#ifndef PKV_PREFILL_PRIO
#define PKV_PREFILL_PRIO 1
#endif
#ifndef PKV_PREFILL_PRIO_QK
#define PKV_PREFILL_PRIO_QK PKV_PREFILL_PRIO
#endif
constexpr int kKBufs = 2;              // K tile buffers in LDS
constexpr int kVBufs = kSkew ? 3 : 2;  // V tile buffers in LDS
constexpr int kXcds = 8;  // accelerator dies (XCDs), each with its own L2

// Column blocks per wave.  (Two, with four waves per workgroup at one wave per
// SIMD, would feed every LDS fragment to two MFMAs, but the accumulators then
// exceed the architectural VGPRs and the code moves them to and from AGPRs.)
constexpr int kNB = 1;
constexpr int kWaves = kCB / kNB;
constexpr int kThreads = 64 * kWaves;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
// Read-only global data seen through the constant address space: uniform
// loads from it are scalar loads (lgkmcnt), which never wait for the vmcnt-
// counted tile copies.
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

// LDS byte address of a shared-memory pointer (the low word of its flat address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8_t*)p;
}

// One direct global -> LDS copy: lane i's 16 bytes at g land at LDS byte
// m0 + 16 i.  Issued through inline asm so that the compiler does not turn it
// into a wait for every in-flight copy before each LDS read; the waits for
// these copies are the explicit vmcnt waits below (vector memory operations
// retire in order).  No memory clobber: every LDS read of a tile buffer is
// separated from the copies into that buffer by a workgroup barrier (a
// compiler fence too), and without it the block-table reads stay scalar loads.
// An LDS-DMA instruction needs one wait state after an SALU write of m0 (the
// s_nop).  m0 is reserved by the compiler, which keeps no value in it in this
// file (a build test checks that every m0 write in the kernels is one of these).
__device__ __forceinline__ void copy_to_lds(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "m0");
}
// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the scalar-base form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0) : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int HW, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int QP = 32 * (kCB / HW);  // positions (members) per workgroup
  constexpr int KSTEPS = D / 16;       // contraction steps of Q K^T
  constexpr int MD = D / 32;           // 32-row blocks of O^T
  constexpr int ROWB = 2 * D;          // bytes per K/V row in LDS
  constexpr int CPR = D / 8;           // 16-byte slots per row
  constexpr int TILEB = kKT * ROWB;    // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;     // rows per copy instruction (4 or 8)
  constexpr int RW = kKT / kWaves;     // rows of each tile copied by one wave
  constexpr int IPW = RW / RPI;        // copy instructions per wave, tile and tensor
  // K tile buffers, then V tile buffers (160 KiB for D = 128 with the skew)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(kKBufs + kVBufs) * TILEB];

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
  int hg;
  if constexpr (SHARED) {
    hg = id % NHG;
    id /= NHG;
  }
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
    // Workgroups are dispatched to the 8 XCDs round-robin (block B on XCD
    // B % 8), each XCD with its own L2.  The query tiles of one (sequence, head
    // group) pair are placed on one XCD at consecutive slots, so the workgroups
    // that run there together read the same K/V tiles through that L2.
    const int xcd = id % kXcds;
    const int slot = id / kXcds;
    const int pair = (slot / a.tiles_per_pair) * kXcds + xcd;
    if (pair >= a.num_seqs * NHG) return;
    const int tile_rev = slot % a.tiles_per_pair;
    hg = pair % NHG;
    b = pair / NHG;
    q0 = a.cu_seqlens_q[b];
    Lq = a.cu_seqlens_q[b + 1] - q0;
    k0 = a.cu_seqlens_k[b];
    Lk = a.cu_seqlens_k[b + 1] - k0;
    const int n_qt = (Lq + QP - 1) / QP;
    tile = n_qt - 1 - tile_rev;  // tiles with the most keys are dispatched first
    if (tile < 0) return;
  }
  const int g = (hg * HW) / G;
  // Positions are relative to key_base.  Prefill: query i sits at shift + i.
  // Shared: every column sees the whole chunk, as a query at its last key.
  const int shift = Lk - Lq;

  // column block nb of this wave: head h[nb], queries (members) first[nb] + col
  int first[kNB], pos[kNB], min_pos[kNB];
  bool col_valid[kNB];
  int64_t q_row[kNB];  // row of q[., Hq, D] (times Hq, plus the head)
  int w_max_pos = -1;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int cb = kNB * wave + nb;
    const int h = hg * HW + cb % HW;
    first[nb] = tile * QP + 32 * (cb / HW);
    const int qi = first[nb] + col;
    col_valid[nb] = qi < Lq;
    pos[nb] = (col_valid[nb] && !SHARED) ? shift + qi : Lk - 1;
    min_pos[nb] = SHARED ? Lk - 1 : shift + first[nb];
    if (first[nb] < Lq) w_max_pos = max(w_max_pos, SHARED ? Lk - 1 : shift + min(first[nb] + 32, Lq) - 1);
    if constexpr (SHARED) {
      q_row[nb] = col_valid[nb] ? (int64_t)a.group_seqs[member0 + qi] * Hq + h : 0;
    } else {
      q_row[nb] = (int64_t)(q0 + qi) * Hq + h;
    }
  }
  const int wg_max_pos = SHARED ? Lk - 1 : shift + min(tile * QP + QP, Lq) - 1;
  const int n_kt = wg_max_pos / kKT + 1;
  const int n_kt_wave = w_max_pos >= 0 ? min(n_kt, w_max_pos / kKT + 1) : 0;

  // Tile copies.  Wave w copies rows RW w .. RW w + RW - 1 of each K and V tile
  // (IPW instructions each, RPI rows per instruction); lane L of an
  // instruction fills slot L % CPR of row L / CPR.  Rows past the end of the
  // sequence re-read the last key's row: their scores are masked (key > every
  // position) and their weights are exactly 0, so finite data suffices.
  const_i32_t* table =
      a.block_tables ? (const_i32_t*)(a.block_tables + (int64_t)b * a.max_blocks_per_seq) : nullptr;
  const int lbs = a.log2_block_size;
  const int bs_mask = (1 << lbs) - 1;
  const uint8_t* kbytes = (const uint8_t*)a.k;
  const uint8_t* vbytes = (const uint8_t*)a.v;
  const int last_key = Lk - 1;
  const int64_t row_bytes = (int64_t)Hkv * ROWB;
  const int64_t blk_bytes = row_bytes << lbs;
  const int64_t head_bytes = (int64_t)g * ROWB;
  const int lr = lane / CPR;
  const int ls = lane % CPR;
  // rows RW w + 8 j .. + 7 lie in one block (block_size >= 8): its id, per group j
  // of 8 rows (the same block for both groups of 16 rows unless block_size is 8)
  constexpr int NBLK = RW / 8;
  int32_t blk[NBLK];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) blk[j] = 0;
  auto fetch_blocks = [&](int t) __attribute__((always_inline)) {
    if (!table) return;
#pragma unroll
    for (int j = 0; j < NBLK; ++j)
      blk[j] = table[uniform((key_base + min(t * kKT + RW * wave + 8 * j, last_key)) >> lbs)];
  };
  // rotation (in 16-byte slots) of V row k: the four rows of one transposing
  // read land in four distinct 64-byte quarters of the 256-byte bank line
  auto vrot = [](int k) __attribute__((always_inline)) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); };
  // Per-lane part of copy instruction i's source (the same for every tile):
  // row lr of the instruction's RPI rows, the KV head, the rotated slot.
  uint32_t lane_src[2 * IPW];
#pragma unroll
  for (int i = 0; i < 2 * IPW; ++i) {
    const int rt = RW * wave + (i % IPW) * RPI + lr;
    const int ch = i >= IPW ? (ls - vrot(rt)) & (CPR - 1) : (ls - rt) & (CPR - 1);
    lane_src[i] = (uint32_t)(lr * row_bytes + head_bytes) + 16 * ch;
  }
  // copy instruction i of tile t into its buffers: K rows for i < IPW, then V
  // rows.  The RPI rows of one instruction start at a multiple of RPI, so they
  // lie in one block; on a tile that reaches past the last key (whose rows
  // then clamp to it) each lane computes its own row.
  auto issue_copy = [&](int t, int vb, int i, bool whole) __attribute__((always_inline)) {
    const int ii = i % IPW;
    const bool is_v = i >= IPW;
    const int bi = is_v ? kKBufs + vb : (t & 1);
    const uint32_t dst = uniform(lds_addr(&lds[bi * TILEB]) + RW * wave * ROWB + ii * 1024);
    const uint8_t* src = is_v ? vbytes : kbytes;
    if (whole) {
      const int r0 = t * kKT + RW * wave + ii * RPI;  // first row of the instruction
      const int64_t row0 = table ? (int64_t)blk[(ii * RPI) / 8] * blk_bytes + (int64_t)((key_base + r0) & bs_mask) * row_bytes
                                 : (int64_t)(k0 + r0) * row_bytes;
      copy_to_lds(src + row0, lane_src[i], dst);
    } else {
      const int rt = RW * wave + ii * RPI + lr;  // row within the tile
      const int tc = min(t * kKT + rt, last_key);
      const int64_t row = table ? (int64_t)blk[(ii * RPI) / 8] * blk_bytes + (int64_t)((key_base + tc) & bs_mask) * row_bytes
                                : (int64_t)(k0 + tc) * row_bytes;
      const int ch = is_v ? (ls - vrot(rt)) & (CPR - 1) : (ls - rt) & (CPR - 1);
      copy_to_lds(src + row + head_bytes + 16 * ch, dst);
    }
  };
  auto issue_copies = [&](int t, int vb) __attribute__((always_inline)) {
    // every row this wave copies of tile t exists
    if (t * kKT + RW * wave + RW - 1 <= last_key) {
#pragma unroll
      for (int i = 0; i < 2 * IPW; ++i) issue_copy(t, vb, i, true);
    } else {
#pragma unroll
      for (int i = 0; i < 2 * IPW; ++i) issue_copy(t, vb, i, false);
    }
  };

  // Fragment read offsets within a tile buffer.
  // K (A operand of S^T): lane (col, half), step kk: key row col (+ 32 mb, which
  // keeps the rotation), chunk 2 kk + half.
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = col * ROWB + 16 * ((2 * kk + half + col) & (CPR - 1));
  // V^T (A operand of O^T), transposing read: lane L = 16 grp + r supplies the
  // 8-byte row of key 8 s + 4 half + r / 4 of a 16-key step (the MFMA's key
  // order) at dims 32 md + 16 (grp % 2) + 4 (r % 4) .. +3, which is chunk
  // 4 md + 2 (grp % 2) + (r % 4) / 2 at byte 8 (r % 2) of it.
  uint32_t voff[MD];
  {
    const int r = lane & 15;
    const int grp = lane >> 4;
    const int qr = 2 * (grp & 1) + (r & 3) / 2 + vrot(r >> 2);
#pragma unroll
    for (int md = 0; md < MD; ++md)
      voff[md] = (4 * half + (r >> 2)) * ROWB + 16 * ((4 * md + qr) & (CPR - 1)) + 8 * (r & 1);
  }

  // Q^T as the B operand: lane (col, half) holds Q[col][16 kk + 8 half .. +8].
  bf16x8_t qf[kNB][KSTEPS];
  f32x16_t acc_o[kNB][MD];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[nb][md][r] = 0.f;
  float m[kNB], lsum[kNB];  // running reference max (log2 units) and this half-wave's weight sum, per column
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m[nb] = kNegInf;
    lsum[nb] = 0.f;
  }
  const float c = a.scale_log2;  // > 0
  const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

  // Scheduling groups (instruction classes of __builtin_amdgcn_sched_group_barrier).
  constexpr int kSchedMfma = 0x008;
  constexpr int kSchedDsRead = 0x100;
  constexpr int kKR = kKB * KSTEPS;  // K fragment reads per tile
  constexpr int kKPF = PKV_PREFILL_KPF;  // K fragment reads in flight
  constexpr int kVR = kKT / 16 * MD;  // V^T fragments per tile (two transposing reads each)
  constexpr int kVPF = PKV_PREFILL_VPF;  // V^T fragments in flight

  // fragment i of K in buffer kb: step kk = i / kKB, key block mb = i % kKB
  auto k_frag = [&](int kb, int i) __attribute__((always_inline)) {
    return __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(&lds[kb * TILEB] + koff[i / kKB] + (i % kKB) * 32 * ROWB));
  };
  // fragment j of V^T in V buffer vb: key step ks = j / MD, dim block md = j % MD
  auto v_frag = [&](int vb, int j) __attribute__((always_inline)) {
    const uint8_t* vp = &lds[(kKBufs + vb) * TILEB] + voff[j % MD] + (j / MD) * 16 * ROWB;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vp));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vp + 8 * ROWB));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8_t vf[kVR];            // V^T fragments (kVPF + 1 live at a time)
  uint32_t pw[kNB][kKT / 4];   // the tile's weights P^T as bf16 pairs

  // S^T = K Q^T (raw scores) for K buffer kb, then the online softmax, which
  // leaves the bf16 weights in pw.  Each K fragment feeds the kNB column
  // blocks, and the reads run kKPF fragments ahead of the MFMAs.  With PRE,
  // the first V^T fragments of V buffer vb are requested at the end of the
  // products, so that they arrive during the softmax.
  auto qk_softmax = [&](int kb, int key0, int vb, auto PRE) __attribute__((always_inline)) {
    constexpr bool pre = decltype(PRE)::value;
    f32x16_t acc_s[kNB][kKB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int mb = 0; mb < kKB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[nb][mb][r] = 0.f;
    bf16x8_t kf[kKR];
    if constexpr (PKV_PREFILL_PRIO_QK > 0) __builtin_amdgcn_s_setprio(PKV_PREFILL_PRIO_QK);
#pragma unroll
    for (int i = 0; i < kKPF; ++i) kf[i] = k_frag(kb, i);
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      if (i + kKPF < kKR) kf[i + kKPF] = k_frag(kb, i + kKPF);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc_s[nb][i % kKB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[nb][i / kKB], acc_s[nb][i % kKB], 0, 0, 0);
    }
    if constexpr (pre) {
#pragma unroll
      for (int j = 0; j < kVPF; ++j) vf[j] = v_frag(vb, j);
    }
#pragma unroll
    for (int i = 0; i < kKPF; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      if (i + kKPF < kKR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kNB, 0);
    }
    if constexpr (pre) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVPF, 0);
    if constexpr (PKV_PREFILL_PRIO_QK > 0) __builtin_amdgcn_s_setprio(0);

#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      // causal mask (only on tiles that reach past the block's first position):
      // key key0 + off(r) with off(r) = mb*32 + (r/4)*8 + half*4 + r%4 is
      // visible iff off(r) - half*4 <= pos - key0 - half*4
      if (key0 + kKT - 1 > min_pos[nb]) {
        const int lim = pos[nb] - key0 - half * 4;
#pragma unroll
        for (int mb = 0; mb < kKB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb * 32 + (r >> 2) * 8 + (r & 3) > lim) acc_s[nb][mb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < kKB; ++mb)
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
      // P^T = 2^(c s - m), rounded to bf16, as the B operand of the 16-key steps
#pragma unroll
      for (int i = 0; i < kKT / 4; ++i) {
        const float s0 = acc_s[nb][i >> 3][(2 * i) & 15];
        const float s1 = acc_s[nb][i >> 3][(2 * i + 1) & 15];
        pw[nb][i] = pack_bf16x2(exp2_hw(fmaf(s0, c, -m[nb])), exp2_hw(fmaf(s1, c, -m[nb])));
        lsum[nb] = dot2_bf16(pw[nb][i], kOnes, lsum[nb]);
      }
    }
  };

  // O^T += V^T P^T for V buffer vb; each V^T fragment feeds the kNB column
  // blocks, read kVPF fragments ahead (the first ones already requested with PRE).
  auto pv = [&](int vb, auto PRE) __attribute__((always_inline)) {
    constexpr bool pre = decltype(PRE)::value;
    if constexpr (PKV_PREFILL_PRIO > 0) __builtin_amdgcn_s_setprio(PKV_PREFILL_PRIO);
    if constexpr (!pre) {
#pragma unroll
      for (int j = 0; j < kVPF; ++j) vf[j] = v_frag(vb, j);
    }
#pragma unroll
    for (int j = 0; j < kVR; ++j) {
      if (j + kVPF < kVR) vf[j + kVPF] = v_frag(vb, j + kVPF);
      const int ks = j / MD, md = j % MD;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const bf16x8_t bf = __builtin_bit_cast(
            bf16x8_t, make_uint4(pw[nb][4 * ks], pw[nb][4 * ks + 1], pw[nb][4 * ks + 2], pw[nb][4 * ks + 3]));
        acc_o[nb][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], bf, acc_o[nb][md], 0, 0, 0);
      }
    }
    if constexpr (!pre) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVPF, 1);
#pragma unroll
    for (int j = 0; j < kVR; ++j) {
      if (j + kVPF < kVR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kNB, 1);
    }
    if constexpr (PKV_PREFILL_PRIO > 0) __builtin_amdgcn_s_setprio(0);
  };

  // Q^T first: its loads are in flight while the first block ids (scalar
  // loads) arrive and the first tile's copies are issued
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const uint16_t* qp = (const uint16_t*)a.q + q_row[nb] * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (col_valid[nb]) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[nb][kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  fetch_blocks(0);
  issue_copies(0, 0);
  if (n_kt > 1) fetch_blocks(1);

  // The compiler's own wait for these loads happens here, once: inside the
  // loop it would also wait for every tile copy in flight.
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) asm volatile("" ::"v"(qf[nb][kk]));
  // Pipeline: tile kt+1 is in flight (direct to LDS) while tile kt is
  // computed; one barrier per tile.  At the barrier of tile kt each wave has
  // waited for its own copies of tile kt (the only ones in flight) and every
  // wave has finished its work on the buffers that the copies of tile kt+1
  // overwrite: K of tile kt-1, and V of tile kt-1 (two buffers) or of tile
  // kt-2 (three buffers, where the late waves still read V of tile kt-1 after
  // the barrier).
  // V buffers of tiles kt - 1, kt and kt + 1 (rotated each tile, no modulo)
  auto tile_loop = [&](auto LATE) __attribute__((always_inline)) {
    constexpr bool is_late = decltype(LATE)::value;
    int vprev = kVBufs - 1, vcur = 0, vnext = 1 % kVBufs;
    for (int kt = 0; kt < n_kt; ++kt) {
      wait_vmem<0>();
      __syncthreads();
      if (kt + 1 < n_kt) issue_copies(kt + 1, vnext);
      if constexpr (is_late) {
        if (kt >= 1 && kt <= n_kt_wave) pv(vprev, std::false_type{});
        if (kt < n_kt_wave) qk_softmax(kt & 1, kt * kKT, 0, std::false_type{});
      } else {
        if (kt < n_kt_wave) {
          qk_softmax(kt & 1, kt * kKT, vcur, std::true_type{});
          pv(vcur, std::true_type{});
        }
      }
      // the next block ids arrive while this wave waits at the next barrier
      if (kt + 2 < n_kt) fetch_blocks(kt + 2);
      const int v_free = vprev;
      vprev = vcur;
      vcur = vnext;
      vnext = kVBufs == 3 ? v_free : vprev;
    }
    // a late wave's last tile (no copies are in flight any more)
    if constexpr (is_late)
      if (n_kt_wave == n_kt && n_kt > 0) pv(vprev, std::false_type{});
  };
  if (kSkew && wave >= kWaves / 2)
    tile_loop(std::true_type{});
  else
    tile_loop(std::false_type{});

  if (n_kt_wave == 0) return;
  if constexpr (SHARED) {
    // unnormalised state of each column at slot slot0 + chunk of its member's pair
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
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
  for (int nb = 0; nb < kNB; ++nb) {
    const float l = halves_sum(lsum[nb]);
    if (!col_valid[nb]) continue;
    const float inv = 1.0f / l;
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

// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides the group size.
int heads_per_wg(int32_t num_q_heads, int32_t num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

template <bool SHARED>
hipError_t launch(const PrefillArgs& a, int32_t head_dim, int64_t blocks, int HW, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(kThreads);
#define PKV_PREFILL_CASE(DD, HH)                                                                     \
  if (head_dim == DD && HW == HH) {                                                                  \
    hipLaunchKernelGGL((prefill_mfma_kernel<DD, HH, SHARED>), grid, block, 0, stream, a);            \
    return hipGetLastError();                                                                        \
  }
  PKV_PREFILL_CASE(128, 8)
  PKV_PREFILL_CASE(128, 4)
  PKV_PREFILL_CASE(128, 2)
  PKV_PREFILL_CASE(128, 1)
  PKV_PREFILL_CASE(64, 8)
  PKV_PREFILL_CASE(64, 4)
  PKV_PREFILL_CASE(64, 2)
  PKV_PREFILL_CASE(64, 1)
#undef PKV_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int HW = heads_per_wg(a.num_q_heads, a.num_kv_heads);
  const int QP = 32 * (kCB / HW);
  PrefillArgs b = a;
  b.tiles_per_pair = (a.max_seqlen_q + QP - 1) / QP;
  const int64_t pairs = (int64_t)a.num_seqs * (a.num_q_heads / HW);
  return launch<false>(b, head_dim, (pairs + kXcds - 1) / kXcds * kXcds * b.tiles_per_pair, HW, stream);
}

int shared_prefix_members_per_wg(int32_t num_q_heads, int32_t num_kv_heads) {
  return 32 * (kCB / heads_per_wg(num_q_heads, num_kv_heads));
}

int64_t shared_prefix_wgs_per_chunk(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_groups,
                                    int32_t max_group_size) {
  const int per_wg = shared_prefix_members_per_wg(num_q_heads, num_kv_heads);
  const int64_t tiles = ((max_group_size > 1 ? max_group_size : 1) + per_wg - 1) / per_wg;
  return (int64_t)num_groups * tiles * (num_q_heads / heads_per_wg(num_q_heads, num_kv_heads));
}

hipError_t launch_shared_prefix_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int HW = heads_per_wg(a.num_q_heads, a.num_kv_heads);
  const int64_t blocks = (int64_t)a.num_groups * a.num_chunks * a.member_tiles * (a.num_q_heads / HW);
  return launch<true>(a, head_dim, blocks, HW, stream);
}

}  // namespace pkv
