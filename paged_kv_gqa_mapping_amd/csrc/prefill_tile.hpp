// Tile machinery of the matrix-core prefill kernels (prefill_mfma.hip): the
// direct global -> LDS copies of K/V tiles, the LDS fragment reads, and one
// wave's two products per tile with the online softmax between them.
//
// A workgroup has 8 waves (two per SIMD) and holds 8 column blocks of 32
// (position, head) columns, one per wave.  K and V tiles of 128 keys are
// staged in LDS once per workgroup, i.e. once for the whole GQA head group.
//
// Tile staging: the copies are direct (global_load_lds_dwordx4: 64 lanes x 16
// bytes per instruction, a wave-uniform base address in SGPRs plus a per-lane
// offset) into tile buffers (two for K, three for V), so that one tile is in
// flight while another is computed, with no register staging.  K and V are
// stored row-major (one row per key, no padding); the 16-byte slot that holds
// chunk c of key row k is rotated by the key (K: (c + k) mod D/8; V: (c + 4
// (k mod 4)) mod 16 for D = 128, (c + 4 (k / 2 mod 2)) mod 8 for D = 64), which
// keeps the fragment reads free of bank conflicts.
//
// Per tile and wave, with v_mfma_f32_32x32x16_bf16:
//   S^T[key][col] = K_tile * Q^T     (4 key blocks x D/16 steps, ds_read_b128)
//   online softmax per column: the accumulator gives each lane one column and
//   16 keys per key block, so the column max and sum are in-lane plus one
//   half-wave exchange;
//   O^T[d][col] += V^T * P^T         (D/32 blocks x 8 steps of 16 keys), where P^T is the
//   S^T accumulator itself, rounded to bf16.  The lane/register layout of an
//   MFMA result is that of its B operand up to a fixed permutation of the 16
//   keys of each step; the V^T fragments are read with ds_read_b64_tr_b16
//   (a transposing LDS read: in each 16-lane group, lane l receives element
//   l % 4 of the 8-byte rows addressed by lanes l / 4 + 4 j, j = 0..3) with
//   row addresses chosen in that permuted key order, so no data moves between
//   lanes.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace pf {

// Keys per tile: 128 (4.4 % faster than 64: half the waits, barriers and copy
// issues per key); one tile's copies are in flight while another is
// computed, ahead by a tile's compute time.
constexpr int kKT = 128;
constexpr int kKB = kKT / 32;  // 32-key blocks per tile
static_assert(kKB == 4, "the softmax joins four per-block chains");
constexpr int kCB = 8;         // column blocks per workgroup
// Skewed schedule: waves 4-7 (which share SIMDs with waves 0-3) multiply a
// tile's weights by V one tile later, after the next barrier, so that the two
// waves of a SIMD are in different phases (one on the matrix core, the other
// in the softmax) instead of in the same one.  V then needs a third buffer.
#ifndef PKV_PREFILL_SKEW
#define PKV_PREFILL_SKEW 1
#endif
constexpr bool kSkew = PKV_PREFILL_SKEW != 0;
// Ping-pong schedule (one-launch and shared-prefix kernels): each tile has two
// segments split by barriers; on every SIMD one wave runs its matrix products
// while the other runs its softmax and issues its copies, and the roles swap
// at the next segment.
#ifndef PKV_PREFILL_PINGPONG
#define PKV_PREFILL_PINGPONG 0
#endif
constexpr bool kPingPong = PKV_PREFILL_PINGPONG != 0;
static_assert(!kPingPong || kSkew, "the ping-pong schedule keeps three V tile buffers");
// With a workspace (a device-side plan of the work): one persistent workgroup
// per CU walking its die's list as one stream of tiles (1), or one workgroup
// per item of the lists, dispatched in list order (0).
#ifndef PKV_PREFILL_PERSISTENT
#define PKV_PREFILL_PERSISTENT 0
#endif
constexpr bool kPlanPersistent = PKV_PREFILL_PERSISTENT != 0;
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
constexpr int kWaves = kCB;
constexpr int kThreads = 64 * kWaves;
// Tile copies: the 128 rows of a tile are 4 row groups of 32; wave w copies
// row group w % 4 of the V tile (waves 0-3) or of the K tile (waves 4-7).
// The skewed loop relies on it: the early waves (0-3) are the V copiers.
constexpr int kRowGroups = 4;
static_assert(kWaves == 2 * kRowGroups, "early waves copy V rows, late waves K rows");

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

template <int D>
struct Geom {
  static constexpr int KSTEPS = D / 16;               // contraction steps of Q K^T
  static constexpr int MD = D / 32;                   // 32-row blocks of O^T
  static constexpr int ROWB = 2 * D;                  // bytes per K/V row in LDS
  static constexpr int CPR = D / 8;                   // 16-byte slots per row
  static constexpr int TILEB = kKT * ROWB;            // bytes per K (or V) tile
  static constexpr int RPI = 1024 / ROWB;             // rows per copy instruction (4 or 8)
  static constexpr int RW = kKT / kRowGroups;         // rows of a tile copied by one wave (its row group)
  static constexpr int IPW = RW / RPI;                // copy instructions per wave and tile
  static constexpr int NBLK = RW / 8;                 // block ids per wave and tile (groups of 8 rows)
  static constexpr int KR = kKB * KSTEPS;             // K fragment reads per tile
  static constexpr int VR = kKT / 16 * MD;            // V^T fragments per tile (two transposing reads each)
  static constexpr int LDS_BYTES = (kKBufs + kVBufs) * TILEB;
};

// rotation (in 16-byte slots) of V row k: the four rows of one transposing
// read land in four distinct 64-byte quarters of the 256-byte bank line
template <int D>
__device__ __forceinline__ int vrot(int k) {
  return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

// Per-wave, per-lane constants: the LDS offsets of the fragment reads and the
// item-independent part of each copy instruction's per-lane source offset.
template <int D>
struct Lanes {
  using Gm = Geom<D>;
  int wave, lane, col, half;
  int rgroup;  // row group this wave copies
  bool vpart;  // it copies V rows (else K rows)
  uint32_t koff[Gm::KSTEPS];
  uint32_t voff[Gm::MD];
  uint32_t src[Gm::IPW];  // row within the instruction (times the row pitch, added per item) and rotated slot

  __device__ __forceinline__ void init(int32_t num_kv_heads) {
    const int tid = threadIdx.x;
    // wave-uniform (scalar): the tile loop bounds and the block-id lookups derive from it
    wave = uniform(tid >> 6);
    lane = tid & 63;
    col = lane & 31;
    half = lane >> 5;
    rgroup = wave % kRowGroups;
    vpart = wave < kRowGroups;
    // K (A operand of S^T): lane (col, half), step kk: key row col (+ 32 mb, which
    // keeps the rotation), chunk 2 kk + half.
#pragma unroll
    for (int kk = 0; kk < Gm::KSTEPS; ++kk)
      koff[kk] = col * Gm::ROWB + 16 * ((2 * kk + half + col) & (Gm::CPR - 1));
    // V^T (A operand of O^T), transposing read: lane L = 16 grp + r supplies the
    // 8-byte row of key 8 s + 4 half + r / 4 of a 16-key step (the MFMA's key
    // order) at dims 32 md + 16 (grp % 2) + 4 (r % 4) .. +3, which is chunk
    // 4 md + 2 (grp % 2) + (r % 4) / 2 at byte 8 (r % 2) of it.
    {
      const int r = lane & 15;
      const int grp = lane >> 4;
      const int qr = 2 * (grp & 1) + (r & 3) / 2 + vrot<D>(r >> 2);
#pragma unroll
      for (int md = 0; md < Gm::MD; ++md)
        voff[md] = (4 * half + (r >> 2)) * Gm::ROWB + 16 * ((4 * md + qr) & (Gm::CPR - 1)) + 8 * (r & 1);
    }
    // copy instruction i fills row lr of its RPI rows, slot ls of the row,
    // holding the rotated chunk ch
    const int lr = lane / Gm::CPR;
    const int ls = lane % Gm::CPR;
    const uint32_t row_bytes = (uint32_t)num_kv_heads * Gm::ROWB;
#pragma unroll
    for (int i = 0; i < Gm::IPW; ++i) {
      const int rt = Gm::RW * rgroup + i * Gm::RPI + lr;
      const int ch = vpart ? (ls - vrot<D>(rt)) & (Gm::CPR - 1) : (ls - rt) & (Gm::CPR - 1);
      src[i] = lr * row_bytes + 16 * ch;
    }
  }
};

// a hook that does nothing
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// One wave's copies of one tile: where every row the wave copies exists
// (`whole`), the byte offsets (in the pool, head included) of its groups of 8
// rows, each group in one block, and issue(i) issues copy instruction i from
// them with two scalar additions; otherwise the copies were issued when the
// tile was planned and issue(i) does nothing.
template <int D>
struct TileCopy {
  using Gm = Geom<D>;
  int64_t off[Gm::NBLK];
  bool whole;

  // dst: LDS byte address of the wave's rows in the destination buffer
  __device__ __forceinline__ void issue(const PrefillArgs& a, const Lanes<D>& ln, uint32_t dst, int i) const {
    if (!whole) return;
    const uint8_t* bytes = (const uint8_t*)(ln.vpart ? a.v : a.k);
    const int64_t row_bytes = (int64_t)a.num_kv_heads * Gm::ROWB;
    copy_to_lds(bytes + off[(i * Gm::RPI) / 8] + ((i * Gm::RPI) % 8) * row_bytes, ln.src[i], uniform(dst + i * 1024));
  }
};

// Where one item's K/V rows are: through a block table row (paged) or packed
// rows from k0, for the keys [key_base, key_base + last_key + 1) of the
// sequence, of KV head g (all wave-uniform).  Tile t of the item holds its
// keys key_base + 128 t ..; rows past last_key re-read the last key's row
// (their scores are masked and their weights exactly 0, so finite data
// suffices).
template <int D>
struct TileSource {
  using Gm = Geom<D>;
  const_i32_t* table;
  int k0, key_base, last_key, lbs_;
  uint32_t head_bytes;

  __device__ __forceinline__ void init(const PrefillArgs& a, int b, int g, int k0_, int key_base_, int Lk) {
    table = a.block_tables ? (const_i32_t*)(a.block_tables + (int64_t)b * a.max_blocks_per_seq) : nullptr;
    lbs_ = a.log2_block_size;
    k0 = k0_;
    key_base = key_base_;
    last_key = Lk - 1;
    head_bytes = (uint32_t)g * Gm::ROWB;
  }

  // block ids of tile t's rows copied by this wave: rows RW r + 8 j .. + 7 of
  // row group r lie in one block (block_size >= 8), one id per group j of 8 rows
  __device__ __forceinline__ void fetch(int32_t (&blk)[Gm::NBLK], int t, const Lanes<D>& ln, int lbs) const {
    if (!table) return;
#pragma unroll
    for (int j = 0; j < Gm::NBLK; ++j)
      blk[j] = table[uniform((key_base + min(t * kKT + Gm::RW * ln.rgroup + 8 * j, last_key)) >> lbs)];
  }

  // The same block ids, fetched with a vector load into lanes 0 .. NBLK - 1
  // (taken out with take()): vector loads wait on the vector memory counter,
  // while scalar loads share a counter with the LDS reads, so that any
  // fragment read issued after a scalar fetch would wait for it.
  __device__ __forceinline__ int32_t fetch_v(int t, const Lanes<D>& ln) const {
    if (!table) return 0;
    const int j = ln.lane < Gm::NBLK ? ln.lane : 0;
    const int row = key_base + min(t * kKT + Gm::RW * ln.rgroup + 8 * j, last_key);
    return ((const int32_t*)table)[row >> lbs_];
  }
  __device__ __forceinline__ static void take(int32_t (&blk)[Gm::NBLK], int32_t v) {
#pragma unroll
    for (int j = 0; j < Gm::NBLK; ++j) blk[j] = __builtin_amdgcn_readlane(v, j);
  }

  // LDS byte address of this wave's rows in K buffer kb or V buffer vb (its part)
  __device__ __forceinline__ static uint32_t dst_of(uint8_t* lds, const Lanes<D>& ln, int kb, int vb) {
    return lds_addr(&lds[(ln.vpart ? kKBufs + vb : kb) * Gm::TILEB]) + Gm::RW * ln.rgroup * Gm::ROWB;
  }

  // Copies of tile t into K buffer kb or V buffer vb (absolute LDS buffer
  // indices): this wave's row group of its part (IPW instructions of RPI rows;
  // lane L of an instruction fills slot L % CPR of row L / CPR).  The RPI rows
  // of one instruction start at a multiple of RPI, so they lie in one block;
  // on a tile that reaches past the last key (whose rows then clamp to it)
  // each lane computes its own row.
  __device__ __forceinline__ void issue(const PrefillArgs& a, uint8_t* lds, const Lanes<D>& ln,
                                        const int32_t (&blk)[Gm::NBLK], int t, int kb, int vb) const {
    const TileCopy<D> tc = plan(a, lds, ln, blk, t, kb, vb);
    const uint32_t dst = dst_of(lds, ln, kb, vb);
#pragma unroll
    for (int i = 0; i < Gm::IPW; ++i) tc.issue(a, ln, dst, i);
  }

  // The copies of tile t for this wave.  Where every row the wave copies
  // exists, they are left to TileCopy::issue; a tile that reaches past the
  // last key is copied here, with per-lane row addresses.
  __device__ __forceinline__ TileCopy<D> plan(const PrefillArgs& a, uint8_t* lds, const Lanes<D>& ln,
                                              const int32_t (&blk)[Gm::NBLK], int t, int kb, int vb) const {
    TileCopy<D> tc;
    const int lbs = a.log2_block_size;
    const int bs_mask = (1 << lbs) - 1;
    const int64_t row_bytes = (int64_t)a.num_kv_heads * Gm::ROWB;
    const int r0 = t * kKT + Gm::RW * ln.rgroup;  // first row (in the item) this wave copies
    tc.whole = r0 + Gm::RW - 1 <= last_key;
    // rows r0 + 8 j .. + 7: one block, consecutive rows in it
#pragma unroll
    for (int j = 0; j < Gm::NBLK; ++j) {
      const int rj = r0 + 8 * j;
      const int64_t row = table ? ((int64_t)blk[j] << lbs) + ((key_base + rj) & bs_mask) : (int64_t)(k0 + rj);
      tc.off[j] = row * row_bytes + head_bytes;
    }
    if (tc.whole) return tc;
    const int lr = ln.lane / Gm::CPR;
    const int ls = ln.lane % Gm::CPR;
    const int64_t blk_bytes = row_bytes << lbs;
    const uint32_t dst = dst_of(lds, ln, kb, vb);
    const uint8_t* bytes = (const uint8_t*)(ln.vpart ? a.v : a.k);
#pragma unroll
    for (int i = 0; i < Gm::IPW; ++i) {
      const int rt = Gm::RW * ln.rgroup + i * Gm::RPI + lr;  // row within the tile
      const int tcl = min(t * kKT + rt, last_key);
      const int64_t row = table ? (int64_t)blk[(i * Gm::RPI) / 8] * blk_bytes +
                                      (int64_t)((key_base + tcl) & bs_mask) * row_bytes
                                : (int64_t)(k0 + tcl) * row_bytes;
      const int ch = ln.vpart ? (ls - vrot<D>(rt)) & (Gm::CPR - 1) : (ls - rt) & (Gm::CPR - 1);
      copy_to_lds(bytes + row + head_bytes + 16 * ch, uniform(dst + i * 1024));
    }
    return tc;
  }
};

// One wave's column block: its queries Q^T, output accumulators O^T, running
// reference max (log2 units) and this half-wave's weight sum, and the tile's
// weights P^T as bf16 pairs; plus the two per-tile phases.
template <int D>
struct WaveTile {
  using Gm = Geom<D>;
  bf16x8_t qf[Gm::KSTEPS];   // Q^T as the B operand: lane (col, half) holds Q[col][16 kk + 8 half .. +8]
  f32x16_t acc_o[Gm::MD];
  float m, lsum;
  uint32_t pw[kKT / 4];      // the tile's weights P^T as bf16 pairs
  bf16x8_t vf[Gm::VR];       // V^T fragments (VPF + 1 live at a time)

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int md = 0; md < Gm::MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[md][r] = 0.f;
    m = kNegInf;
    lsum = 0.f;
  }

  // Q rows of this wave's columns: q_row = the row of q[., Hq, D] (times Hq,
  // plus the head); invalid columns get zeros.
  __device__ __forceinline__ void load_q(const void* q, int64_t q_row, bool valid, int half) {
    const uint16_t* qp = (const uint16_t*)q + q_row * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < Gm::KSTEPS; ++kk) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  // make the compiler's wait for the Q loads happen here, once (inside a tile
  // loop it would also wait for every tile copy in flight)
  __device__ __forceinline__ void settle_q() {
#pragma unroll
    for (int kk = 0; kk < Gm::KSTEPS; ++kk) asm volatile("" ::"v"(qf[kk]));
  }

  // fragment i of K in buffer kb: step kk = i / kKB, key block mb = i % kKB
  __device__ __forceinline__ bf16x8_t k_frag(const uint8_t* lds, const Lanes<D>& ln, int kb, int i) const {
    return __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(&lds[kb * Gm::TILEB] + ln.koff[i / kKB] + (i % kKB) * 32 * Gm::ROWB));
  }
  // fragment j of V^T in V buffer vb: key step ks = j / MD, dim block md = j % MD
  __device__ __forceinline__ bf16x8_t v_frag(const uint8_t* lds, const Lanes<D>& ln, int vb, int j) const {
    const uint8_t* vp = &lds[(kKBufs + vb) * Gm::TILEB] + ln.voff[j % Gm::MD] + (j / Gm::MD) * 16 * Gm::ROWB;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vp));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vp + 8 * Gm::ROWB));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // the first V^T fragments of V buffer vb, requested ahead of pv<true>
  __device__ __forceinline__ void prefetch_v(const uint8_t* lds, const Lanes<D>& ln, int vb) {
#pragma unroll
    for (int j = 0; j < PKV_PREFILL_VPF; ++j) vf[j] = v_frag(lds, ln, vb, j);
  }

  // S^T = K Q^T for K buffer kb, then the online softmax (both below).
  template <bool PRE>
  __device__ __forceinline__ void qk_softmax(const uint8_t* lds, const Lanes<D>& ln, int kb, int key0, int vb, int pos,
                                             int min_pos, float c) {
    f32x16_t acc_s[kKB];
    qk<PRE>(lds, ln, kb, vb, acc_s);
    softmax(ln, acc_s, key0, pos, min_pos, c);
  }

  // S^T = K Q^T (raw scores, one 32-key block each) for K buffer kb into acc_s, the K fragment reads
  // kKPF ahead of the MFMAs; with PRE, the first V^T fragments of V buffer vb
  // are requested at the end, so that they arrive during the softmax.
  template <bool PRE>
  __device__ __forceinline__ void qk(const uint8_t* lds, const Lanes<D>& ln, int kb, int vb, f32x16_t (&acc_s)[kKB]) {
    constexpr int kSchedMfma = 0x008;
    constexpr int kSchedDsRead = 0x100;
    constexpr int kKPF = PKV_PREFILL_KPF;
    constexpr int kVPF = PKV_PREFILL_VPF;
#pragma unroll
    for (int mb = 0; mb < kKB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[mb][r] = 0.f;
    bf16x8_t kf[Gm::KR];
    if constexpr (PKV_PREFILL_PRIO_QK > 0) __builtin_amdgcn_s_setprio(PKV_PREFILL_PRIO_QK);
#pragma unroll
    for (int i = 0; i < kKPF; ++i) kf[i] = k_frag(lds, ln, kb, i);
#pragma unroll
    for (int i = 0; i < Gm::KR; ++i) {
      if (i + kKPF < Gm::KR) kf[i + kKPF] = k_frag(lds, ln, kb, i + kKPF);
      acc_s[i % kKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i / kKB], acc_s[i % kKB], 0, 0, 0);
    }
    if constexpr (PRE) {
#pragma unroll
      for (int j = 0; j < kVPF; ++j) vf[j] = v_frag(lds, ln, vb, j);
    }
#pragma unroll
    for (int i = 0; i < kKPF; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
    for (int i = 0; i < Gm::KR; ++i) {
      if (i + kKPF < Gm::KR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    }
    if constexpr (PRE) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVPF, 0);
    if constexpr (PKV_PREFILL_PRIO_QK > 0) __builtin_amdgcn_s_setprio(0);
  }

  // The online softmax of the scores in acc_s (keys key0 ..), which leaves the
  // bf16 weights in pw.  Column position pos sees keys <= pos; the mask is
  // applied only on tiles that reach past the block's first position min_pos.
  // c = scale * log2(e) > 0.
  // hook(i) runs after the weights of keys 4i .. 4i+3 (i < 32) are made: the
  // ping-pong schedule issues its tile copies there, spread over the softmax.
  template <typename Hook = NoHook>
  __device__ __forceinline__ void softmax(const Lanes<D>& ln, f32x16_t (&acc_s)[kKB], int key0, int pos, int min_pos,
                                          float c, const Hook& hook = Hook()) {
    const int half = ln.half;
    // causal mask (only on tiles that reach past the block's first position):
    // key key0 + off(r) with off(r) = mb*32 + (r/4)*8 + half*4 + r%4 is
    // visible iff off(r) - half*4 <= pos - key0 - half*4
    if (key0 + kKT - 1 > min_pos) {
      const int lim = pos - key0 - half * 4;
#pragma unroll
      for (int mb = 0; mb < kKB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
        {
          if (mb * 32 + (r >> 2) * 8 + (r & 3) > lim) acc_s[mb][r] = kNegInf;
          // one compare and select at a time: hoisted together, the 64 lane
          // masks would fill the scalar registers
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the column max, as kKB independent chains (one per key block) joined at the end
    float bmx[kKB];
#pragma unroll
    for (int mb = 0; mb < kKB; ++mb) {
      bmx[mb] = acc_s[mb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bmx[mb] = fmaxf(bmx[mb], acc_s[mb][r]);
    }
    float mx = bmx[0];
#pragma unroll
    for (int mb = 1; mb < kKB; ++mb) mx = fmaxf(mx, bmx[mb]);
    mx = halves_max(mx) * c;  // c > 0, so the max commutes with the scaling
    if (wave_any(mx > m + kTau)) {
      const float mn = fmaxf(m, mx);
      const float alpha = exp2_hw(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int md = 0; md < Gm::MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[md][r] *= alpha;
    }
    // P^T = 2^(c s - m), rounded to bf16, as the B operand of the 16-key steps;
    // the weight sum in kKB independent chains (one per key block), added to
    // the running sum at the end
    const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
    float bl[kKB];
#pragma unroll
    for (int mb = 0; mb < kKB; ++mb) bl[mb] = 0.f;
#pragma unroll
    for (int i = 0; i < kKT / 4; ++i) {
      const float s0 = acc_s[i >> 3][(2 * i) & 15];
      const float s1 = acc_s[i >> 3][(2 * i + 1) & 15];
      pw[i] = pack_bf16x2(exp2_hw(fmaf(s0, c, -m)), exp2_hw(fmaf(s1, c, -m)));
      bl[i >> 3] = dot2_bf16(pw[i], kOnes, bl[i >> 3]);
      hook(i);
    }
    lsum += (bl[0] + bl[1]) + (bl[2] + bl[3]);
  }

  // O^T += V^T P^T for V buffer vb, V^T fragments read kVPF ahead (the first
  // ones already requested with PRE).
  template <bool PRE>
  __device__ __forceinline__ void pv(const uint8_t* lds, const Lanes<D>& ln, int vb) {
    constexpr int kSchedMfma = 0x008;
    constexpr int kSchedDsRead = 0x100;
    constexpr int kVPF = PKV_PREFILL_VPF;
    if constexpr (PKV_PREFILL_PRIO > 0) __builtin_amdgcn_s_setprio(PKV_PREFILL_PRIO);
    if constexpr (!PRE) {
#pragma unroll
      for (int j = 0; j < kVPF; ++j) vf[j] = v_frag(lds, ln, vb, j);
    }
#pragma unroll
    for (int j = 0; j < Gm::VR; ++j) {
      if (j + kVPF < Gm::VR) vf[j + kVPF] = v_frag(lds, ln, vb, j + kVPF);
      const int ks = j / Gm::MD, md = j % Gm::MD;
      const bf16x8_t bf =
          __builtin_bit_cast(bf16x8_t, make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]));
      acc_o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], bf, acc_o[md], 0, 0, 0);
    }
    if constexpr (!PRE) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVPF, 1);
#pragma unroll
    for (int j = 0; j < Gm::VR; ++j) {
      if (j + kVPF < Gm::VR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
    }
    if constexpr (PKV_PREFILL_PRIO > 0) __builtin_amdgcn_s_setprio(0);
  }

  // the column's normalised output rounded to bf16, stored for a valid column
  // (every lane takes part in the half-wave sum)
  __device__ __forceinline__ void store_out(void* out, int64_t q_row, int half, bool valid) const {
    const float l = halves_sum(lsum);
    if (!valid) return;
    const float inv = 1.0f / l;
    uint16_t* op = (uint16_t*)out + q_row * D + half * 4;
#pragma unroll
    for (int md = 0; md < Gm::MD; ++md) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rr * 4;
        uint2 w;
        w.x = pack_bf16x2(acc_o[md][r] * inv, acc_o[md][r + 1] * inv);
        w.y = pack_bf16x2(acc_o[md][r + 2] * inv, acc_o[md][r + 3] * inv);
        *reinterpret_cast<uint2*>(op + md * 32 + rr * 8) = w;
      }
    }
  }
};

}  // namespace pf
}  // namespace pkv
