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
//
// PERSIST mode is the persistent prefill: kPersistWgs workgroups, each on
// die blockIdx % 8, take items (a query tile and a range of its key tiles)
// from that die's list, written by the plan kernel (prefill_plan.hip); the
// first item of a workgroup is given by its index, the next one is claimed
// from the die's queue head while the current one runs.  An item that is a
// whole query tile writes the output; a piece of a split query tile writes
// its unnormalised state (m, l, o) to its slot, counts itself in the tile's
// arrival counter, and the piece that arrives last merges the states of all
// pieces in piece order (so the bits do not depend on which piece was last)
// with M = max m_j, out = sum 2^(m_j - M) o_j / sum 2^(m_j - M) l_j.
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

enum Mode { kGrid = 0, kShared = 1, kPersist = 2 };

// One work item of a workgroup.  Prefill: query tile `tile` of sequence b
// (Lq queries from packed row q0, Lk keys from packed row k0), key tiles
// [kt_lo, kt_hi) (kt_hi < 0: all it needs).  Shared: member tile `tile` of a
// group (Lq members from member0), keys [key_base, key_base + Lk) of its
// prefix, table row b.  Persistent pieces: piece `piece` of `pieces`, arrival
// counter `split` (< 0: a whole query tile), state slots from `slot`.
struct Item {
  int b, hg, tile, q0, Lq, k0, Lk, key_base, member0, chunk;
  int kt_lo, kt_hi, piece, pieces, split, slot;
  long long* tl;  // timeline record of this item (PKV_PREFILL_TIMELINE builds), or NULL
};

// timeline stamp (a diagnostic of the persistent kernel; compiled out by default)
__device__ __forceinline__ void stamp(const Item& it, int field) {
#ifdef PKV_PREFILL_TIMELINE
  if (it.tl && threadIdx.x == 0) it.tl[field] = wall_clock64();
#else
  (void)it;
  (void)field;
#endif
}

// A piece of a split query tile: write this piece's state (per wave and
// lane: the O^T accumulators, the reference max m and the column's weight
// sum l) to its slot, count the piece in the tile's arrival counter, and if
// it is the last to arrive, merge every piece's state in piece order and
// write the output rows.
//
// All pieces of a query tile sit in one die's list, and list x is worked by
// the workgroups w with w % 8 == x, which the dispatcher places on one die
// (round-robin over the dies of the partition: die w % 8 on a full chip, as
// read back from the die id register of every workgroup), so the states,
// the counter and the merger share one L2 and need no device-wide cache
// maintenance: each wave waits until its state
// stores are acknowledged by the L2 (the vector L1 writes through) before
// the workgroup barrier, the count is an L2 atomic, and the merger's loads
// miss its L1 (a slot is written once per launch and read once, by the
// merger; the L1 is invalidated when a launch starts).
template <int D>
__device__ __forceinline__ void merge_pieces(const PrefillArgs& a, uint8_t* lds, const Item& it,
                                             const f32x16_t* acc, float m, float l, bool valid, int64_t q_row) {
  constexpr int MD = D / 32;
  constexpr int NR = MD * 16 + 2;  // floats per lane of a wave's state
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t slot_floats = (int64_t)kWaves * NR * 64;
  float* const wbase = a.plan_states + (int64_t)it.slot * slot_floats + (int64_t)wave * NR * 64 + lane;
  auto at = [&](int piece, int r) { return wbase + piece * slot_floats + r * 64; };
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) *at(it.piece, md * 16 + r) = acc[md][r];
  *at(it.piece, MD * 16) = m;
  *at(it.piece, MD * 16 + 1) = l;
  wait_vmem<0>();
  __syncthreads();
  volatile int32_t* flag = reinterpret_cast<volatile int32_t*>(lds);
  if (tid == 0)
    *flag = __hip_atomic_fetch_add(a.plan_arrive + it.split, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            it.pieces - 1;
  __syncthreads();
  if (!*flag) return;
  if (!valid) return;
  // M = max_j m_j; L = sum_j 2^(m_j - M) l_j; out = sum_j 2^(m_j - M) o_j / L, in piece order
  float M = kNegInf;
  for (int j = 0; j < it.pieces; ++j) M = fmaxf(M, j == it.piece ? m : *at(j, MD * 16));
  float L = 0.f;
  for (int j = 0; j < it.pieces; ++j) {
    const float mj = j == it.piece ? m : *at(j, MD * 16);
    const float lj = j == it.piece ? l : *at(j, MD * 16 + 1);
    L = fmaf(exp2_hw(mj - M), lj, L);
  }
  const float inv = 1.0f / L;
  const int half = lane >> 5;
  uint16_t* op = (uint16_t*)a.out + q_row * D + half * 4;
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] = 0.f;
    for (int j = 0; j < it.pieces; ++j) {
      const float w = exp2_hw((j == it.piece ? m : *at(j, MD * 16)) - M);
      if (j == it.piece) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = fmaf(w, acc[md][r], o[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = fmaf(w, *at(j, md * 16 + r), o[r]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = rr * 4;
      uint2 w;
      w.x = pack_bf16x2(o[r] * inv, o[r + 1] * inv);
      w.y = pack_bf16x2(o[r + 2] * inv, o[r + 3] * inv);
      *reinterpret_cast<uint2*>(op + md * 32 + rr * 8) = w;
    }
  }
}

template <int D, int HW, int MODE>
__device__ __forceinline__ void run_item(const PrefillArgs& a, uint8_t* lds, const Item& it) {
  constexpr bool SHARED = MODE == kShared;
  constexpr int QP = 32 * (kCB / HW);  // positions (members) per workgroup
  constexpr int KSTEPS = D / 16;       // contraction steps of Q K^T
  constexpr int MD = D / 32;           // 32-row blocks of O^T
  constexpr int ROWB = 2 * D;          // bytes per K/V row in LDS
  constexpr int CPR = D / 8;           // 16-byte slots per row
  constexpr int TILEB = kKT * ROWB;    // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;     // rows per copy instruction (4 or 8)
  constexpr int RW = kKT / kWaves;     // rows of each tile copied by one wave
  constexpr int IPW = RW / RPI;        // copy instructions per wave, tile and tensor

  const int tid = threadIdx.x;
  // wave-uniform (scalar): the tile loop bounds and the block-id lookups derive from it
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int b = it.b, hg = it.hg, tile = it.tile, q0 = it.q0, Lq = it.Lq, k0 = it.k0, Lk = it.Lk;
  const int key_base = it.key_base, member0 = it.member0, chunk = it.chunk;
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
  // key tiles [kt_lo, n_kt) of this item; this wave computes [kt_lo, n_kt_wave)
  const int kt_lo = it.kt_lo;
  const int n_kt = it.kt_hi >= 0 ? it.kt_hi : wg_max_pos / kKT + 1;
  const int n_kt_wave = w_max_pos >= 0 ? min(n_kt, w_max_pos / kKT + 1) : kt_lo;

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
  fetch_blocks(kt_lo);
  issue_copies(kt_lo, 0);
  if (kt_lo + 1 < n_kt) fetch_blocks(kt_lo + 1);

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
    for (int kt = kt_lo; kt < n_kt; ++kt) {
      wait_vmem<0>();
      __syncthreads();
      if (kt == kt_lo) stamp(it, 5);
      if (kt + 1 < n_kt) issue_copies(kt + 1, vnext);
      if constexpr (is_late) {
        if (kt >= kt_lo + 1 && kt <= n_kt_wave) pv(vprev, std::false_type{});
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
      if (n_kt_wave == n_kt && n_kt > kt_lo) pv(vprev, std::false_type{});
  };
  if (kSkew && wave >= kWaves / 2)
    tile_loop(std::true_type{});
  else
    tile_loop(std::false_type{});

  stamp(it, 6);
  if constexpr (MODE == kPersist) {
    if (it.split >= 0) {
      merge_pieces<D>(a, lds, it, acc_o[0], m[0], halves_sum(lsum[0]), col_valid[0] && n_kt_wave > kt_lo,
                      q_row[0]);
      return;
    }
  }
  if (n_kt_wave == kt_lo) return;
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

template <int D, int HW, int MODE>
__global__ __launch_bounds__(kThreads, 1) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int QP = 32 * (kCB / HW);
  // K tile buffers, then V tile buffers (160 KiB for D = 128 with the skew)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(kKBufs + kVBufs) * kKT * 2 * D];
  const int NHG = a.num_q_heads / HW;
  if constexpr (MODE == kShared) {
    Item it{};
    it.kt_hi = -1;
    it.split = -1;
    int id = blockIdx.x;
    it.hg = id % NHG;
    id /= NHG;
    it.tile = id % a.member_tiles;
    id /= a.member_tiles;
    it.chunk = id % a.num_chunks;
    const int gi = id / a.num_chunks;
    it.member0 = a.group_offsets[gi];
    it.Lq = a.group_offsets[gi + 1] - it.member0;
    if (it.tile * QP >= it.Lq) return;
    it.b = a.group_seqs[it.member0];
    const int shared = a.shared_lens[it.b];
    it.key_base = it.chunk * a.chunk_tokens;
    if (it.key_base >= shared) return;
    it.Lk = min(shared - it.key_base, a.chunk_tokens);
    run_item<D, HW, MODE>(a, lds, it);
  } else if constexpr (MODE == kGrid) {
    // Workgroups are dispatched to the 8 XCDs round-robin (block B on XCD
    // B % 8), each XCD with its own L2.  The query tiles of one (sequence, head
    // group) pair are placed on one XCD at consecutive slots, so the workgroups
    // that run there together read the same K/V tiles through that L2.
    Item it{};
    it.kt_hi = -1;
    it.split = -1;
    const int id = blockIdx.x;
    const int xcd = id % kXcds;
    const int slot = id / kXcds;
    const int pair = (slot / a.tiles_per_pair) * kXcds + xcd;
    if (pair >= a.num_seqs * NHG) return;
    const int tile_rev = slot % a.tiles_per_pair;
    it.hg = pair % NHG;
    it.b = pair / NHG;
    it.q0 = a.cu_seqlens_q[it.b];
    it.Lq = a.cu_seqlens_q[it.b + 1] - it.q0;
    it.k0 = a.cu_seqlens_k[it.b];
    it.Lk = a.cu_seqlens_k[it.b + 1] - it.k0;
    const int n_qt = (it.Lq + QP - 1) / QP;
    it.tile = n_qt - 1 - tile_rev;  // tiles with the most keys are dispatched first
    if (it.tile < 0) return;
    run_item<D, HW, MODE>(a, lds, it);
  } else {
    // the die's list; the first item by workgroup index, the next ones from the
    // die's queue head (claimed at the start of the current item)
    const int xcd = blockIdx.x % kPlanXcds;
    const_i32_t* hdr = (const_i32_t*)a.plan_hdr;
    const int count = min(hdr[kPlanXcds + xcd], a.items_cap);
    int idx = blockIdx.x / kPlanXcds;
#ifdef PKV_PREFILL_TIMELINE
    int n_items = 0;
    long long t_item = wall_clock64();
#endif
    while (idx < count) {
      int next = 0;
      if (threadIdx.x == 0)
        next = __hip_atomic_fetch_add(a.plan_queue + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const_i32_t* rec = (const_i32_t*)a.plan_items + ((int64_t)xcd * a.items_cap + idx) * kItemInts;
      Item it{};
      it.b = rec[kItB];
      it.hg = rec[kItHg];
      it.tile = rec[kItTile];
      it.kt_lo = rec[kItKtLo];
      it.kt_hi = rec[kItKtHi];
      it.piece = rec[kItChunk] & 0xffff;
      it.pieces = rec[kItChunk] >> 16;
      it.split = rec[kItSplit];
      it.slot = rec[kItSlot];
      const_i32_t* cq = (const_i32_t*)a.cu_seqlens_q;
      const_i32_t* ck = (const_i32_t*)a.cu_seqlens_k;
      it.q0 = cq[it.b];
      it.Lq = cq[it.b + 1] - it.q0;
      it.k0 = ck[it.b];
      it.Lk = ck[it.b + 1] - it.k0;
#ifdef PKV_PREFILL_TIMELINE
      if (a.timeline && n_items < kTimelineItems) {
        it.tl = a.timeline + ((int64_t)blockIdx.x * kTimelineItems + n_items) * kTimelineFields;
        if (threadIdx.x == 0) {
          it.tl[0] = idx | ((long long)xcd << 32);
          it.tl[1] = it.b | ((long long)it.hg << 16) | ((long long)it.tile << 32);
          it.tl[2] = it.kt_lo | ((long long)it.kt_hi << 32);
          it.tl[3] = it.piece | ((long long)it.pieces << 16) | ((long long)(it.split + 1) << 32);
          it.tl[4] = t_item;
        }
      }
      ++n_items;
#endif
      run_item<D, HW, MODE>(a, lds, it);
      // every wave is done with the tile buffers before the next item's copies
      __syncthreads();
      stamp(it, 7);
      if (threadIdx.x == 0) *reinterpret_cast<volatile int32_t*>(lds) = next;
      __syncthreads();
      idx = uniform(*reinterpret_cast<volatile int32_t*>(lds));
#ifdef PKV_PREFILL_TIMELINE
      t_item = wall_clock64();
#endif
    }
#ifdef PKV_PREFILL_TIMELINE
    if (a.timeline && n_items < kTimelineItems && threadIdx.x == 0)
      a.timeline[((int64_t)blockIdx.x * kTimelineItems + n_items) * kTimelineFields] = -1;  // end of this list
#endif
  }
}

// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides the group size.
int heads_per_wg(int32_t num_q_heads, int32_t num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

template <int MODE>
hipError_t launch(const PrefillArgs& a, int32_t head_dim, int64_t blocks, int HW, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(kThreads);
#define PKV_PREFILL_CASE(DD, HH)                                                                     \
  if (head_dim == DD && HW == HH) {                                                                  \
    hipLaunchKernelGGL((prefill_mfma_kernel<DD, HH, MODE>), grid, block, 0, stream, a);              \
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
  if (a.plan_hdr) return launch<kPersist>(a, head_dim, kPersistWgs, HW, stream);
  const int QP = 32 * (kCB / HW);
  PrefillArgs b = a;
  b.tiles_per_pair = (a.max_seqlen_q + QP - 1) / QP;
  const int64_t pairs = (int64_t)a.num_seqs * (a.num_q_heads / HW);
  return launch<kGrid>(b, head_dim, (pairs + kXcds - 1) / kXcds * kXcds * b.tiles_per_pair, HW, stream);
}

int prefill_tile_positions(int32_t num_q_heads, int32_t num_kv_heads) {
  return 32 * (kCB / heads_per_wg(num_q_heads, num_kv_heads));
}

int prefill_head_groups(int32_t num_q_heads, int32_t num_kv_heads) {
  return num_q_heads / heads_per_wg(num_q_heads, num_kv_heads);
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
  return launch<kShared>(a, head_dim, blocks, HW, stream);
}

}  // namespace pkv
