// Causal varlen prefill attention on the gfx950 matrix cores (bf16 operands,
// fp32 accumulation), over paged or packed K/V; the tile machinery (copies,
// fragment reads, the two products and the online softmax) is in
// prefill_tile.hpp.
//
// Work split: a workgroup (8 waves, two per SIMD) takes one sequence, one group
// of HW query heads that share a KV head, and QP = 32 * (8 / HW) consecutive
// query positions (a query tile): 8 column blocks of 32 (position, head)
// columns, wave w holding head w % HW and positions 32 * (w / HW) .. +31 of the
// tile.  It walks the key axis in tiles of 128 keys up to its last query's
// position.  Query i of a sequence sits at position Lk - Lq + i and sees keys
// <= it; the mask is applied only on tiles that reach past a column block's
// first position.
//
// Three kernels:
//  * GRID: one workgroup per query tile, one launch.  The query tiles of one
//    (sequence, head group) pair run back to back on one XCD, so that they
//    share the K/V tiles through its L2.
//  * SHARED: the group pass of shared-prefix ("cascade") decode: the columns
//    are the decode queries of the members of one group (sequences whose first
//    keys are the same cached blocks), the keys one chunk of that shared
//    prefix, with no causal mask (every member's token comes after the prefix),
//    and the result is each column's unnormalised softmax state (m, l, o)
//    written to the member's decode workspace, merged later with the states of
//    its own keys.  The shared keys are thus read once per group instead of
//    once per member.
//  * STREAM (persistent): kPersistWgs workgroups, workgroup w on die w % 8,
//    work through the items of that die's list (written by the plan kernel,
//    prefill_plan.hip): an item is a query tile and a range of its key tiles.
//    The workgroup treats its items as one stream of tiles: the copies of the
//    next tile, the block ids of the one after it and the next item's queries
//    are issued while the current tile is computed, whether or not they belong
//    to the next item, so an item costs no prologue of its own.  The previous
//    item's output (and, for the waves that run late, its last P V product) is
//    finished at the top of the next item's first tile.  The items are known
//    two ahead: a workgroup takes its first kPlanStaticItems items by its index,
//    and at the start of each item wave 0 claims one more from the die's queue
//    head and publishes it in a mailbox word of the workgroup when the item
//    ends, for the other waves to read during the next item's first tile.
//    A whole query tile writes its output; a piece of a split query tile writes
//    its unnormalised state (m, l, o) to its slot and counts itself in the
//    tile's arrival counter, and the piece that arrives last merges the states
//    of all pieces in piece order (so the bits do not depend on which piece was
//    last) with M = max m_j, out = sum 2^(m_j - M) o_j / sum 2^(m_j - M) l_j.
//    Each wave merges its own columns, with its own arrival counter.
#include "prefill_tile.hpp"

namespace pkv {

using namespace pf;

namespace {

enum Mode { kGrid = 0, kShared = 1 };

// One work item of the GRID and SHARED kernels.  Prefill: query tile `tile` of
// sequence b (Lq queries from packed row q0, Lk keys from packed row k0).
// Shared: member tile `tile` of a group (Lq members from member0), keys
// [key_base, key_base + Lk) of its prefix, table row b.
struct Item {
  int b, hg, tile, q0, Lq, k0, Lk, key_base, member0, chunk;
  // a piece of a planned query tile: key tiles [kt_lo, kt_hi) (kt_hi < 0: all
  // the tile needs); split >= 0: piece pc & 0xffff of pc >> 16, arrival
  // counters from split * 8 and state slots from `slot`
  int kt_lo = 0, kt_hi = -1, split = -1, slot = 0, pc = 0;
};

// record idx of die xcd's list
__device__ __forceinline__ const_i32_t* item_record(const PrefillArgs& a, int xcd, int idx) {
  return (const_i32_t*)a.plan_items + ((int64_t)xcd * a.items_cap + idx) * kItemInts;
}

// A piece of a split query tile, one wave's columns: write the state (the O^T
// accumulators, the reference max m and the column's weight sum l) to its
// slot, count the wave's part of the piece in its arrival counter, and if it
// is the last of the pieces to arrive, merge every piece's state in piece
// order and write the output rows.
//
// All pieces of a query tile sit in one die's list, and list x is worked by
// the workgroups w with w % 8 == x, which the dispatcher places on one die
// (round-robin over the dies of the partition: die w % 8 on a full chip, as
// read back from the die id register of every workgroup), so the states, the
// counter and the merger share one L2 and need no device-wide cache
// maintenance: the wave waits until its state stores are acknowledged by the
// L2 (the vector L1 writes through) before it counts, the count is an L2
// atomic, and the merger's loads miss its L1 (a slot is written once per
// launch and read once, by the merger; the L1 is invalidated when a launch
// starts).  This runs before the next tile's copies are issued, so the wait
// covers only the state stores.
template <int D>
__device__ __forceinline__ void finish_piece(const PrefillArgs& a, int split, int slot, int piece, int pieces,
                                             int64_t q_row, const WaveTile<D>& wt, int wave, int lane) {
  using Gm = Geom<D>;
  constexpr int NR = Gm::MD * 16 + 2;  // floats per lane of a wave's state
  const int64_t slot_floats = (int64_t)kWaves * NR * 64;
  float* const wbase = a.plan_states + (int64_t)slot * slot_floats + (int64_t)wave * NR * 64 + lane;
  auto at = [&](int j, int r) { return wbase + j * slot_floats + r * 64; };
  const float l = halves_sum(wt.lsum);
#pragma unroll
  for (int md = 0; md < Gm::MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) *at(piece, md * 16 + r) = wt.acc_o[md][r];
  *at(piece, Gm::MD * 16) = wt.m;
  *at(piece, Gm::MD * 16 + 1) = l;
  wait_vmem<0>();
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(a.plan_arrive + split * kWaves + wave, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::: "memory");  // the other pieces' states are read after the count
  if (uniform(old) != pieces - 1) return;
  // M = max_j m_j; L = sum_j 2^(m_j - M) l_j; out = sum_j 2^(m_j - M) o_j / L, in piece order
  float M = kNegInf;
  for (int j = 0; j < pieces; ++j) M = fmaxf(M, j == piece ? wt.m : *at(j, Gm::MD * 16));
  float L = 0.f;
  for (int j = 0; j < pieces; ++j) {
    const float mj = j == piece ? wt.m : *at(j, Gm::MD * 16);
    const float lj = j == piece ? l : *at(j, Gm::MD * 16 + 1);
    L = fmaf(exp2_hw(mj - M), lj, L);
  }
  if (q_row < 0) return;
  const float inv = 1.0f / L;
  const int half = lane >> 5;
  uint16_t* op = (uint16_t*)a.out + q_row * D + half * 4;
#pragma unroll
  for (int md = 0; md < Gm::MD; ++md) {
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] = 0.f;
    for (int j = 0; j < pieces; ++j) {
      const float w = exp2_hw((j == piece ? wt.m : *at(j, Gm::MD * 16)) - M);
      if (j == piece) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = fmaf(w, wt.acc_o[md][r], o[r]);
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
  using Gm = Geom<D>;
  constexpr bool SHARED = MODE == kShared;
  constexpr int QP = 32 * (kCB / HW);  // positions (members) per workgroup
  Lanes<D> ln;
  ln.init(a.num_kv_heads);
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int g = (it.hg * HW) / G;
  // Positions are relative to key_base.  Prefill: query i sits at shift + i.
  // Shared: every column sees the whole chunk, as a query at its last key.
  const int shift = it.Lk - it.Lq;
  // this wave's column block: head h, queries (members) first + col
  const int h = it.hg * HW + ln.wave % HW;
  const int first = it.tile * QP + 32 * (ln.wave / HW);
  const int qi = first + ln.col;
  const bool col_valid = qi < it.Lq;
  const int pos = (col_valid && !SHARED) ? shift + qi : it.Lk - 1;
  const int min_pos = SHARED ? it.Lk - 1 : shift + first;
  const int w_max_pos = first < it.Lq ? (SHARED ? it.Lk - 1 : shift + min(first + 32, it.Lq) - 1) : -1;
  // row of q[., Hq, D] (times Hq, plus the head) of query (member) q of this
  // wave's head; computed again after the tile loop rather than kept live
  auto row_of = [&](int q) -> int64_t {
    if constexpr (SHARED)
      return q < it.Lq ? (int64_t)a.group_seqs[it.member0 + q] * Hq + h : 0;
    else
      return (int64_t)(it.q0 + q) * Hq + h;
  };
  const int wg_max_pos = SHARED ? it.Lk - 1 : shift + min(it.tile * QP + QP, it.Lq) - 1;
  // key tiles [kt0, n_kt) of this item; this wave computes [kt0, n_kt_wave)
  const int kt0 = it.kt_lo;
  const int n_kt = it.kt_hi >= 0 ? it.kt_hi : wg_max_pos / kKT + 1;
  const int n_kt_wave = w_max_pos >= 0 ? min(n_kt, w_max_pos / kKT + 1) : kt0;

  const int lbs = a.log2_block_size;
  TileSource<D> src;
  src.init(a, it.b, g, it.k0, it.key_base, it.Lk);
  int32_t blk[Gm::NBLK];
#pragma unroll
  for (int j = 0; j < Gm::NBLK; ++j) blk[j] = 0;
  WaveTile<D> wt;
  wt.reset();
  const float c = a.scale_log2;  // > 0

  // Q^T first: its loads are in flight while the first block ids (scalar
  // loads) arrive and the first tile's copies are issued
  wt.load_q(a.q, row_of(qi), col_valid, ln.half);
  src.fetch(blk, kt0, ln, lbs);
  src.issue(a, lds, ln, blk, kt0, 0, 0);
  // block ids of the next tile: vector-loaded for the one-barrier loop
  // (taken out after the next barrier), scalar-loaded for the ping-pong loop
  int32_t vblk = 0;
  if (kt0 + 1 < n_kt) {
    if (!kPingPong)
      vblk = src.fetch_v(kt0 + 1, ln);
    else
      src.fetch(blk, kt0 + 1, ln, lbs);
  }
  wt.settle_q();

  // Pipeline: tile kt+1 is in flight (direct to LDS) while tile kt is
  // computed; one barrier per tile.  At the barrier of tile kt each wave has
  // waited for its own copies of tile kt (the only ones in flight) and every
  // wave has finished its work on the buffers that the copies of tile kt+1
  // overwrite: K of tile kt-1, and V of tile kt-1 (two buffers) or of tile
  // kt-2 (three buffers, where the late waves still read V of tile kt-1 after
  // the barrier).  V buffers of tiles kt - 1, kt and kt + 1 rotate each tile.
  auto tile_loop = [&](auto LATE) __attribute__((always_inline)) {
    constexpr bool is_late = decltype(LATE)::value;
    int vprev = kVBufs - 1, vcur = 0, vnext = 1 % kVBufs;
    for (int kt = kt0; kt < n_kt; ++kt) {
      const int kb = (kt - kt0) & 1;  // K buffer of tile kt
      wait_vmem<0>();
      __syncthreads();
      if (kt + 1 < n_kt) {
        // tile kt+1's block ids arrived with this barrier's wait; tile kt+2's
        // are requested before its copies (the next barrier's wait covers them)
        TileSource<D>::take(blk, vblk);
        if (kt + 2 < n_kt) vblk = src.fetch_v(kt + 2, ln);
      }
      if constexpr (is_late) {
        // the late waves copy K rows, which the next tile needs first: at
        // once, after requesting the first V^T fragments of their P V (LDS
        // reads, which do not wait for the copies to pass the address path)
        const bool do_pv = kt > kt0 && kt <= n_kt_wave;
        if (do_pv) wt.prefetch_v(lds, ln, vprev);
        if (kt + 1 < n_kt) src.issue(a, lds, ln, blk, kt + 1, kb ^ 1, vnext);
        if (do_pv) wt.template pv<true>(lds, ln, vprev);
        if (kt < n_kt_wave) wt.template qk_softmax<false>(lds, ln, kb, kt * kKT, 0, pos, min_pos, c);
      } else {
        // the early waves copy V rows, needed only by the next tile's P V:
        // after their Q K^T, so that the tile starts with matrix products
        // while the late waves' copies pass the address path
        f32x16_t acc_s[kKB];
        if (kt < n_kt_wave) wt.template qk<true>(lds, ln, kb, vcur, acc_s);
        if (kt + 1 < n_kt) src.issue(a, lds, ln, blk, kt + 1, kb ^ 1, vnext);
        if (kt < n_kt_wave) {
          wt.softmax(ln, acc_s, kt * kKT, pos, min_pos, c);
          wt.template pv<true>(lds, ln, vcur);
        }
      }
      const int v_free = vprev;
      vprev = vcur;
      vcur = vnext;
      vnext = kVBufs == 3 ? v_free : vprev;
    }
    // a late wave's last tile (no copies are in flight any more)
    if constexpr (is_late)
      if (n_kt_wave == n_kt && n_kt > kt0) wt.template pv<false>(lds, ln, vprev);
  };
  // Ping-pong: waves 0-3 (group E, one per SIMD) and 4-7 (group L) alternate
  // between their products and their softmax, so that in each segment one
  // wave of a SIMD keeps its matrix core busy while the other computes the
  // exponentials.  Tile kt:
  //   segment A: E: O^T += V(kt-1) P(kt-1)^T, S(kt) = K(kt) Q^T;
  //              L: softmax of S(kt-1), then the copies of K(kt+1)
  //   segment B: E: softmax of S(kt), then the copies of V(kt+1);
  //              L: O^T += V(kt-1) P(kt-1)^T, S(kt) = K(kt) Q^T
  // with one more tile (kt = n_kt) for the last P V product.  K tiles use two
  // buffers (K(kt+1) goes where K(kt-1) was, whose readers finished before
  // barrier A of tile kt), V tiles three (V(kt+1) goes where V(kt-2) was).
  // At barrier A each L wave has waited for its copies of K(kt) and each E
  // wave for its copies of V(kt-1) (those of V(kt), issued one segment later,
  // may still be in flight: vector memory operations complete in order).
  // The two groups run separate copies of the loop (the same barriers in the
  // same order), so that each keeps only its own values live.
  auto pingpong = [&](auto GROUP_E) __attribute__((always_inline)) {
    constexpr bool is_e = decltype(GROUP_E)::value;
    f32x16_t acc_s[kKB];
    int vprev = kVBufs - 1, vnext = 1 % kVBufs;  // V buffers of tiles kt-1 and kt+1
    auto copies = [&](int kt) __attribute__((always_inline)) {
      if (kt + 1 < n_kt) {
        src.issue(a, lds, ln, blk, kt + 1, (kt + 1 - kt0) & 1, vnext);
        if (kt + 2 < n_kt) src.fetch(blk, kt + 2, ln, lbs);
      }
    };
    auto products = [&](int kt) __attribute__((always_inline)) {
      if (kt > kt0 && kt - 1 < n_kt_wave) wt.template pv<false>(lds, ln, vprev);
      if (kt < n_kt_wave) wt.template qk<false>(lds, ln, (kt - kt0) & 1, 0, acc_s);
    };
    for (int kt = kt0; kt <= n_kt; ++kt) {
      if (is_e && kt > kt0 && kt < n_kt)
        wait_vmem<Gm::IPW>();
      else
        wait_vmem<0>();
      __syncthreads();
      if constexpr (is_e) {
        products(kt);
      } else {
        if (kt > kt0 && kt - 1 < n_kt_wave) wt.softmax(ln, acc_s, (kt - 1) * kKT, pos, min_pos, c);
        copies(kt);
      }
      __syncthreads();
      if constexpr (is_e) {
        if (kt < n_kt_wave) wt.softmax(ln, acc_s, kt * kKT, pos, min_pos, c);
        copies(kt);
      } else {
        products(kt);
      }
      // V buffers: tile kt's becomes the previous one, tile kt+2's takes the
      // oldest (that of tile kt-1)
      const int v_kt = vprev == kVBufs - 1 ? 0 : vprev + 1;
      vnext = vprev;
      vprev = v_kt;
    }
  };
  if (kPingPong && ln.vpart)
    pingpong(std::true_type{});
  else if (kPingPong)
    pingpong(std::false_type{});
  else if (kSkew && ln.wave >= kWaves / 2)
    tile_loop(std::true_type{});
  else
    tile_loop(std::false_type{});

  if (n_kt_wave <= kt0) return;
  // this lane's column from the lane id (two instructions) instead of a
  // register held through the loop
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int half_e = lane_e >> 5;
  const int qi_e = first + (lane_e & 31);
  const int64_t q_row = row_of(qi_e);
  const bool col_valid_e = qi_e < it.Lq;
  if constexpr (SHARED) {
    // unnormalised state of each column at slot slot0 + chunk of its member's pair
    const float l = halves_sum(wt.lsum);
    if (!col_valid_e) return;
    const int64_t slot = q_row * a.ws_stride + a.slot0 + it.chunk;
    float* wo = a.ws_o + slot * D + half_e * 4;
#pragma unroll
    for (int md = 0; md < Gm::MD; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rr * 4;
        *reinterpret_cast<float4*>(wo + md * 32 + rr * 8) =
            make_float4(wt.acc_o[md][r], wt.acc_o[md][r + 1], wt.acc_o[md][r + 2], wt.acc_o[md][r + 3]);
      }
    if (half_e == 0) {
      a.ws_ml[slot * 2] = wt.m;
      a.ws_ml[slot * 2 + 1] = l;
    }
  } else if (it.split < 0) {
    wt.store_out(a.out, q_row, half_e, col_valid_e);
  } else {
    finish_piece<D>(a, it.split, it.slot, it.pc & 0xffff, it.pc >> 16, col_valid_e ? q_row : -1, wt, ln.wave,
                    ln.lane);
  }
}

template <int D, int HW, int MODE>
__global__ __launch_bounds__(kThreads, 1) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int QP = 32 * (kCB / HW);
  // K tile buffers, then V tile buffers (160 KiB for D = 128 with the skew)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Geom<D>::LDS_BYTES];
  const int NHG = a.num_q_heads / HW;
  Item it{};
  if constexpr (MODE == kShared) {
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
  } else {
    // Workgroups are dispatched to the 8 XCDs round-robin (block B on XCD
    // B % 8), each XCD with its own L2.  The query tiles of one (sequence, head
    // group) pair are placed on one XCD at consecutive slots, so the workgroups
    // that run there together read the same K/V tiles through that L2.
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
  }
  run_item<D, HW, MODE>(a, lds, it);
}

// ---------------------------------------------------------------- planned grid

// One workgroup per item of the plan's lists (workgroup w takes item w / 8 of
// die w % 8's list; the dispatcher places it on that die): the query tiles
// with their long key ranges cut into pieces, the largest pairs first, so
// that the dispatcher's own order balances the dies' workgroups.  Pieces of a
// split query tile are merged by the last to arrive, as in the persistent
// kernel.
template <int D, int HW>
__global__ __launch_bounds__(kThreads, 1) void prefill_items_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Geom<D>::LDS_BYTES];
  const int xcd = blockIdx.x % kPlanXcds;
  const int idx = blockIdx.x / kPlanXcds;
  const_i32_t* hdr = (const_i32_t*)a.plan_hdr;
  // a plan that overflowed its lists left holes in them (the host sizes the
  // lists so that this cannot happen)
  if (idx >= min(hdr[kPlanXcds + xcd], a.items_cap) || hdr[kHdrOverflow] != 0) return;
  const_i32_t* rec = item_record(a, xcd, idx);
  Item it{};
  it.b = rec[kItB];
  it.hg = rec[kItHg];
  it.tile = rec[kItTile];
  it.kt_lo = rec[kItKtLo];
  it.kt_hi = rec[kItKtHi];
  it.pc = rec[kItChunk];
  it.split = rec[kItSplit];
  it.slot = rec[kItSlot];
  const_i32_t* cq = (const_i32_t*)a.cu_seqlens_q;
  const_i32_t* ck = (const_i32_t*)a.cu_seqlens_k;
  it.q0 = cq[it.b];
  it.Lq = cq[it.b + 1] - it.q0;
  it.k0 = ck[it.b];
  it.Lk = ck[it.b + 1] - it.k0;
  run_item<D, HW, kGrid>(a, lds, it);
}

// ---------------------------------------------------------------- persistent stream

// The kernel's arguments, read from the kernel argument segment where this is
// called.  The persistent kernel's scalar registers are too few to hold every
// argument across its loop, so the ones used once per item are loaded again
// at each use (the empty asm makes the pointer opaque, so that the loads are
// neither hoisted out of the loop nor merged).
__device__ __forceinline__ const PrefillArgs& args_here() {
  typedef const __attribute__((address_space(4))) PrefillArgs const_args_t;
  const_args_t* p = (const_args_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const PrefillArgs*)p;
}

// The part of an item the stream keeps in scalar registers: its key tiles
// [kt_lo, kt_hi), and for this wave the block's first position and the end of
// the key tiles it computes; per lane, each column's row of q and out (times
// Hq, plus the head; -1 past the queries).  Column col's position is
// min_pos + col (past the sequence's queries the column's output is not
// written, so its position does not matter).  The rest of the record (piece,
// split) is read again when the item ends.
struct Item2 {
  int kt_lo, kt_hi, min_pos, n_kt_wave;
  int64_t q_row;
  __device__ __forceinline__ bool valid() const { return q_row >= 0; }
};

// Item idx of die xcd's list: what the stream keeps of it, and where its K/V rows are.
template <int D, int HW>
__device__ __forceinline__ void load_item(const PrefillArgs& a, int xcd, int idx, int wave, int col, Item2& x,
                                          TileSource<D>& src) {
  constexpr int QP = 32 * (kCB / HW);
  const_i32_t* rec = item_record(a, xcd, idx);
  const int b = rec[kItB];
  const int hg = rec[kItHg];
  const int tile = rec[kItTile];
  x.kt_lo = rec[kItKtLo];
  x.kt_hi = rec[kItKtHi];
  const_i32_t* cq = (const_i32_t*)a.cu_seqlens_q;
  const_i32_t* ck = (const_i32_t*)a.cu_seqlens_k;
  const int q0 = cq[b];
  const int Lq = cq[b + 1] - q0;
  const int k0 = ck[b];
  const int Lk = ck[b + 1] - k0;
  const int Hq = a.num_q_heads;
  src.init(a, b, (hg * HW) / (Hq / a.num_kv_heads), k0, 0, Lk);
  const int head = hg * HW + wave % HW;
  const int first = tile * QP + 32 * (wave / HW);
  const int qi = first + col;
  const int shift = Lk - Lq;
  const bool valid = qi < Lq;
  x.q_row = valid ? (int64_t)(q0 + qi) * Hq + head : -1;
  x.min_pos = shift + first;
  const int w_max_pos = first < Lq ? shift + min(first + 32, Lq) - 1 : -1;
  x.n_kt_wave = w_max_pos >= 0 ? min(x.kt_hi, w_max_pos / kKT + 1) : x.kt_lo;
}

// The end of item idx for one wave: its output (if the wave computed any of
// its key tiles), or its state as a piece.
template <int D>
__device__ __forceinline__ void finish_item(const PrefillArgs& a, int xcd, int idx, int64_t q_row, bool computed,
                                            const WaveTile<D>& wt, const Lanes<D>& ln) {
  const_i32_t* rec = item_record(a, xcd, idx);
  const int split = rec[kItSplit];
  if (split < 0) {
    if (computed) wt.store_out(a.out, q_row, ln.half, q_row >= 0);
  } else {
    const int pc = rec[kItChunk];
    finish_piece<D>(a, split, rec[kItSlot], pc & 0xffff, pc >> 16, q_row, wt, ln.wave, ln.lane);
  }
}

// timeline stamps (a diagnostic; compiled in with PKV_PREFILL_TIMELINE only):
// per workgroup and item, fields 0 workgroup | die << 32, 1 kt_lo | kt_hi << 32,
// 2 item index, 4 start, 5 the previous item finished, 6 this item's tiles done
__device__ __forceinline__ void stamp(int n, int field, long long v) {
#ifdef PKV_PREFILL_TIMELINE
  const PrefillArgs& a = args_here();
  if (a.timeline && n < kTimelineItems && threadIdx.x == 0)
    a.timeline[((int64_t)blockIdx.x * kTimelineItems + n) * kTimelineFields + field] = v;
#else
  (void)n;
  (void)field;
  (void)v;
#endif
}
__device__ __forceinline__ long long stamp_now() {
#ifdef PKV_PREFILL_TIMELINE
  return wall_clock64();
#else
  return 0;
#endif
}

template <int D, int HW>
__global__ __launch_bounds__(kThreads, 1) void prefill_stream_kernel(PrefillArgs a) {
  using Gm = Geom<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Gm::LDS_BYTES];
  const int xcd = blockIdx.x % kPlanXcds;
  const int wgi = blockIdx.x / kPlanXcds;  // this workgroup's index on its die
  const_i32_t* hdr = (const_i32_t*)a.plan_hdr;
  const int count = min(hdr[kPlanXcds + xcd], a.items_cap);
  // a plan that overflowed its lists left holes in them (the host sizes the
  // lists so that this cannot happen)
  if (wgi >= count || hdr[kHdrOverflow] != 0) return;
  Lanes<D> ln;
  ln.init(a.num_kv_heads);
  const int lbs = a.log2_block_size;
  const float c = a.scale_log2;  // > 0

  auto stream = [&](auto LATE) __attribute__((always_inline)) {
    constexpr bool is_late = decltype(LATE)::value;
    // the items known ahead: cur (being computed), nxt and the index of the one
    // after it (an index >= count: none)
    int idx_cur = wgi;
    int idx_nxt = wgi + kPlanCusPerXcd;
    int idx_nn = wgi + 2 * kPlanCusPerXcd;
    Item2 cur, nxt;
    TileSource<D> src_cur, src_nxt;
    load_item<D, HW>(args_here(), xcd, idx_cur, ln.wave, ln.col, cur, src_cur);
    nxt = cur;
    src_nxt = src_cur;
    if (idx_nxt < count) load_item<D, HW>(args_here(), xcd, idx_nxt, ln.wave, ln.col, nxt, src_nxt);
    int claimed = 0;  // lane 0 of wave 0: the item claimed for the one after idx_nn
    if (idx_nn < count && threadIdx.x == 0)
      claimed = __hip_atomic_fetch_add(args_here().plan_queue + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Copy cursor: the next tile whose copies are to be issued, key tile ct of
    // item csel (0 cur, 1 nxt, 2 none known yet); blk holds its block ids.
    int32_t blk[Gm::NBLK];
#pragma unroll
    for (int j = 0; j < Gm::NBLK; ++j) blk[j] = 0;
    src_cur.fetch(blk, cur.kt_lo, ln, lbs);
    src_cur.issue(a, lds, ln, blk, cur.kt_lo, 0, 0);
    int csel = 0, ct = cur.kt_lo + 1;
    if (ct >= cur.kt_hi) {
      csel = idx_nxt < count ? 1 : 2;
      ct = nxt.kt_lo;
    }
    auto prefetch_blocks = [&]() __attribute__((always_inline)) {
      if (csel == 0)
        src_cur.fetch(blk, ct, ln, lbs);
      else if (csel == 1)
        src_nxt.fetch(blk, ct, ln, lbs);
    };
    prefetch_blocks();

    WaveTile<D> wt;
    wt.reset();
    wt.load_q(args_here().q, cur.q_row, cur.valid(), ln.half);
    wt.settle_q();

    int gt = 0;  // stream tile counter: K buffer gt & 1
    int vprev = kVBufs - 1, vcur = 0, vnext = 1 % kVBufs;
    // the previous item, finished at the top of the next item's first tile
    int idx_prv = idx_cur;
    int64_t q_row_prv = cur.q_row;
    bool computed_prv = false, late_pv_prv = false;
    int n_item = 0;
    stamp(n_item, 0, (long long)wgi | ((long long)xcd << 32));
    stamp(n_item, 1, (long long)cur.kt_lo | ((long long)cur.kt_hi << 32));
    stamp(n_item, 2, idx_cur);
    stamp(n_item, 4, stamp_now());
    int kt = cur.kt_lo;
    for (;;) {
      wait_vmem<0>();
      __syncthreads();
      if (kt == cur.kt_lo && n_item > 0) {
        // the previous item's end: a late wave's last P V product, then its output or state
        if constexpr (is_late)
          if (late_pv_prv) wt.template pv<false>(lds, ln, vprev);
        finish_item<D>(args_here(), xcd, idx_prv, q_row_prv, computed_prv, wt, ln);
        wt.reset();
        wt.settle_q();  // cur's queries (loaded during the previous item's last tile) are in
        stamp(n_item, 5, stamp_now());
      }
      // copies of the tile after this one in the stream
      if (csel < 2) {
        if (csel == 0)
          src_cur.issue(a, lds, ln, blk, ct, (gt + 1) & 1, vnext);
        else
          src_nxt.issue(a, lds, ln, blk, ct, (gt + 1) & 1, vnext);
        if (++ct >= (csel == 0 ? cur.kt_hi : nxt.kt_hi)) {
          if (csel == 0 && idx_nxt < count) {
            csel = 1;
            ct = nxt.kt_lo;
          } else {
            csel = 2;  // the following item's copies start once it is loaded
          }
        }
      }
      const bool last = kt + 1 >= cur.kt_hi;
      // compute tile kt of cur
      if constexpr (is_late) {
        if (kt > cur.kt_lo && kt <= cur.n_kt_wave) wt.template pv<false>(lds, ln, vprev);
        if (kt < cur.n_kt_wave) wt.template qk_softmax<false>(lds, ln, gt & 1, kt * kKT, 0, cur.min_pos + ln.col, cur.min_pos, c);
      } else {
        if (kt < cur.n_kt_wave) {
          wt.template qk_softmax<true>(lds, ln, gt & 1, kt * kKT, vcur, cur.min_pos + ln.col, cur.min_pos, c);
          if (!last) wt.template pv<true>(lds, ln, vcur);
        }
      }
      // the next item's queries, once this wave's last Q K^T of cur is done
      if (last && idx_nxt < count) wt.load_q(args_here().q, nxt.q_row, nxt.valid(), ln.half);
      if constexpr (!is_late)
        if (last && kt < cur.n_kt_wave) wt.template pv<true>(lds, ln, vcur);
      // block ids of the copy cursor's tile (they arrive while this wave waits at the next barrier)
      prefetch_blocks();
      if (kt == cur.kt_lo && idx_nxt < count && n_item > 0) {
        // the mailbox word that wave 0 published when the previous item ended
        // (before the barrier above) names the item after nxt.  The two words
        // alternate by item: wave 0 may publish this item's word while other
        // waves still read the previous one, but the word it overwrites next
        // was read by every wave before the barrier at the top of that item.
        int v = 0;
        if (ln.lane == 0)
          v = __hip_atomic_fetch_add(args_here().plan_mailbox + 2 * blockIdx.x + ((n_item - 1) & 1), 0,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        idx_nn = uniform(v);
      }
      const int v_free = vprev;
      vprev = vcur;
      vcur = vnext;
      vnext = kVBufs == 3 ? v_free : vprev;
      ++gt;
      if (!last) {
        ++kt;
        continue;
      }
      // cur's tiles are done: wave 0 publishes the item it claimed when cur began
      if (threadIdx.x == 0 && idx_nn < count) args_here().plan_mailbox[2 * blockIdx.x + (n_item & 1)] = claimed;
      stamp(n_item, 6, stamp_now());
      if (idx_nxt >= count) break;
      idx_prv = idx_cur;
      q_row_prv = cur.q_row;
      computed_prv = cur.n_kt_wave > cur.kt_lo;
      late_pv_prv = cur.n_kt_wave == cur.kt_hi && cur.kt_hi > cur.kt_lo;
      idx_cur = idx_nxt;
      cur = nxt;
      src_cur = src_nxt;
      idx_nxt = idx_nn;
      idx_nn = count;  // learned at the end of the new item's first tile
      if (idx_nxt < count) load_item<D, HW>(args_here(), xcd, idx_nxt, ln.wave, ln.col, nxt, src_nxt);
      // the copy cursor was in the old nxt (now cur) or past it
      if (csel == 1) {
        csel = 0;
      } else if (idx_nxt < count) {
        csel = 1;
        ct = nxt.kt_lo;
        prefetch_blocks();
      }
      if (idx_nxt < count && threadIdx.x == 0)
        claimed = __hip_atomic_fetch_add(args_here().plan_queue + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++n_item;
      stamp(n_item, 0, (long long)wgi | ((long long)xcd << 32));
      stamp(n_item, 1, (long long)cur.kt_lo | ((long long)cur.kt_hi << 32));
      stamp(n_item, 2, idx_cur);
      stamp(n_item, 4, stamp_now());
      kt = cur.kt_lo;
    }
    // the last item's end (no copies are in flight any more)
    if constexpr (is_late)
      if (cur.n_kt_wave == cur.kt_hi && cur.kt_hi > cur.kt_lo) wt.template pv<false>(lds, ln, vprev);
    finish_item<D>(args_here(), xcd, idx_cur, cur.q_row, cur.n_kt_wave > cur.kt_lo, wt, ln);
    stamp(n_item + 1, 0, -1);
  };
  if (kSkew && ln.wave >= kWaves / 2)
    stream(std::true_type{});
  else
    stream(std::false_type{});
}

// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides the group size.
int heads_per_wg(int32_t num_q_heads, int32_t num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

template <typename K>
hipError_t launch_kernel(K kernel, int64_t blocks, const PrefillArgs& a, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch(const PrefillArgs& a, int32_t head_dim, int64_t blocks, int HW, hipStream_t stream) {
#define PKV_PREFILL_CASE(DD, HH) \
  if (head_dim == DD && HW == HH) return launch_kernel(prefill_mfma_kernel<DD, HH, MODE>, blocks, a, stream);
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

hipError_t launch_items(const PrefillArgs& a, int32_t head_dim, int HW, hipStream_t stream) {
  const int64_t blocks = (int64_t)kPlanXcds * a.items_cap;
#define PKV_ITEMS_CASE(DD, HH) \
  if (head_dim == DD && HW == HH) return launch_kernel(prefill_items_kernel<DD, HH>, blocks, a, stream);
  PKV_ITEMS_CASE(128, 8)
  PKV_ITEMS_CASE(128, 4)
  PKV_ITEMS_CASE(128, 2)
  PKV_ITEMS_CASE(128, 1)
  PKV_ITEMS_CASE(64, 8)
  PKV_ITEMS_CASE(64, 4)
  PKV_ITEMS_CASE(64, 2)
  PKV_ITEMS_CASE(64, 1)
#undef PKV_ITEMS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const PrefillArgs& a, int32_t head_dim, int HW, hipStream_t stream) {
#define PKV_STREAM_CASE(DD, HH) \
  if (head_dim == DD && HW == HH) return launch_kernel(prefill_stream_kernel<DD, HH>, kPersistWgs, a, stream);
  PKV_STREAM_CASE(128, 8)
  PKV_STREAM_CASE(128, 4)
  PKV_STREAM_CASE(128, 2)
  PKV_STREAM_CASE(128, 1)
  PKV_STREAM_CASE(64, 8)
  PKV_STREAM_CASE(64, 4)
  PKV_STREAM_CASE(64, 2)
  PKV_STREAM_CASE(64, 1)
#undef PKV_STREAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  const int HW = heads_per_wg(a.num_q_heads, a.num_kv_heads);
  if (a.plan_hdr) return kPlanPersistent ? launch_stream(a, head_dim, HW, stream) : launch_items(a, head_dim, HW, stream);
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
