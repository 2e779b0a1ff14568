// Host-side launchers of the device kernels (one per translation unit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

hipError_t launch_kv_store(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                           int64_t num_tokens, int32_t row_bytes, hipStream_t stream);

hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* cu_seqlens_k, int32_t num_seqs,
                         int32_t max_seqlen_k, void* k_out, void* v_out, int32_t row_bytes, int32_t log2_block_size,
                         hipStream_t stream);

// Arguments of the row-attention kernel (decode rows, or prefill rows on the vector path).
struct RowAttnArgs {
  const void* q;            // decode: [B, Hq, D]; prefill: [total_q, Hq, D]
  const void* k;            // paged caches or packed rows
  const void* v;
  const int32_t* block_tables;  // NULL: packed k/v rows (prefill only)
  const int32_t* context_lens;  // decode: [B]
  const int32_t* cu_seqlens_q;  // prefill: [B + 1]
  const int32_t* cu_seqlens_k;  // prefill: [B + 1]
  void* out;
  float* ws_o;   // [B, Hq, ws_stride, D] fp32 partial outputs (decode, S > 1 or shared prefixes)
  float* ws_ml;  // [B, Hq, ws_stride, 2] fp32 (running max in log2 units, sum)
  // Shared-prefix (cascade) decode: sequence b's keys [0, kv_start[b]) are
  // attended by the group pass, which leaves ceil(kv_start[b] / prefix_chunk)
  // states at slots num_splits .. of the pair; the split pass covers the rest.
  const int32_t* kv_start;  // [B] or NULL (no shared prefixes)
  // Decode with the store fused in: sequence b's newest token (position
  // context_lens[b] - 1) is read from k_new/v_new [B, Hkv, D] instead of the
  // cache, and written to its cache row by the wave that reads it.
  const void* k_new;  // NULL: plain decode
  const void* v_new;
  int32_t ws_stride;        // state slots per (sequence, query head): num_splits + prefix chunks
  int32_t prefix_chunk;     // keys per group-pass state
  float scale_log2;  // scale * log2(e)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t log2_block_size;
  int32_t split_tokens;  // decode: tokens per split
  int32_t num_splits;    // decode: S, the split count of the grid (ceil(max_context_len / split_tokens))
  int32_t max_rows;      // prefill: max_seqlen_q
  // Token-balanced decode (balance_pieces = W > 0 instead of fixed splits):
  // sequence b is n_b = max(1, ceil(L_b / U)) steps of U tokens; the N steps
  // of the batch, sequence after sequence, are cut into W' <= W ranges (the
  // launch's waves per KV-head group), nearly equal (row_attn.hpp: the
  // waves on odd-numbered dies take 1/16 less).
  // The part of sequence b in wave w's range writes its states at slot w + b
  // ([w + b, Hq] of ws_o / ws_ml; a sequence's parts have consecutive slots),
  // and the wave holding b's first step writes (first slot, part count) to
  // piece_meta[b].
  // With shared prefixes (kv_start set) each sequence's steps count only its
  // own keys [kv_start[b], L_b), and the group pass's chunk states of pair p
  // sit at rows prefix_slot0 + p * prefix_states + chunk.
  int32_t balance_pieces;
  int32_t* piece_meta;  // [B, 2]
  int64_t prefix_slot0;
  int32_t prefix_states;
};

// Picks the instantiation (dtype, head_dim, KV heads per wave, group size) and launches.
// `prefill` selects prefill rows (causal, one split) instead of decode rows.
hipError_t launch_row_attn(const RowAttnArgs& a, int32_t dtype, int32_t head_dim, bool prefill, hipStream_t stream);

hipError_t launch_decode_reduce(const RowAttnArgs& a, int32_t dtype, int32_t head_dim, hipStream_t stream);

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_tables;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  void* out;
  float scale_log2;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t log2_block_size;
  int32_t max_seqlen_q;
  int32_t tiles_per_pair;  // set by the launcher: query tiles per (sequence, head group)
  // Group pass of shared-prefix decode (q is [B, Hq, D]; NULL group_seqs = prefill):
  // group gi's members are group_seqs[group_offsets[gi] ..], all sharing their
  // first shared_lens[member] keys (same blocks); each workgroup takes up to
  // 32 * (4 / heads per wave) members, one KV head's query heads and one chunk
  // of chunk_tokens keys, and writes that chunk's softmax state per (member,
  // head) at slot slot0 + chunk of the member's decode workspace.
  const int32_t* group_offsets;
  const int32_t* group_seqs;
  const int32_t* shared_lens;
  float* ws_o;
  float* ws_ml;
  int32_t ws_stride;
  int32_t slot0;
  int32_t chunk_tokens;
  int32_t num_groups;
  int32_t num_chunks;     // grid: ceil(max shared length / chunk_tokens)
  int32_t member_tiles;   // grid: ceil(max group size / members per workgroup)
  // Persistent prefill (a workspace was given): the work lists written by
  // the plan kernel, the per-XCD queue heads, arrival counters of split query
  // tiles and their softmax-state slots (offsets of PrefillPlanLayout).
  const int32_t* plan_hdr;
  int32_t* plan_queue;
  const int32_t* plan_items;
  int32_t* plan_arrive;    // per split query tile and wave
  int32_t* plan_mailbox;   // per workgroup, two words: the item index claimed for it, by item parity
  float* plan_states;
  int32_t items_cap;
  // built with PKV_PREFILL_TIMELINE only: per workgroup and item, timestamps
  // of the persistent kernel (a diagnostic; NULL otherwise)
  long long* timeline;
};
// timeline records per workgroup, int64 fields per record
constexpr int kTimelineItems = 64;
constexpr int kTimelineFields = 8;

// ---------------------------------------------------------------- persistent prefill plan
//
// The persistent prefill runs kPersistWgs workgroups, kPlanCusPerXcd on each
// of kPlanXcds accelerator dies; workgroup w runs on die w % kPlanXcds and
// takes work items from that die's list.  An item is one query tile (QP
// positions x the HW query heads of one KV head) of one sequence and a range
// of its 128-key tiles.  A query tile with many keys is cut into several
// items along its keys ("pieces"); each piece writes its unnormalised softmax
// state, and the last piece to finish merges them.
constexpr int kPlanXcds = 8;
constexpr int kPlanCusPerXcd = 32;
constexpr int kPersistWgs = kPlanXcds * kPlanCusPerXcd;
// waves per workgroup of the prefill kernels (each merges its own columns of a split tile)
constexpr int kPlanWaves = 8;
// items a workgroup takes by its index before it claims from the die's queue
// (the next items are known two ahead, so their copies can be issued early)
constexpr int kPlanStaticItems = 3;
// pieces are at least kPlanMinCap key tiles; the cap is chosen so that each
// die's list holds about kPlanItemsPerCu maximal pieces per workgroup
#ifndef PKV_PLAN_ITEMS_PER_CU
#define PKV_PLAN_ITEMS_PER_CU 3
#endif
constexpr int kPlanMinCap = 4;
constexpr int kPlanItemsPerCu = PKV_PLAN_ITEMS_PER_CU;
constexpr int kPlanThreads = 1024;
// sequences a plan holds in LDS; a call with more runs the one-launch kernel
constexpr int kPlanMaxSeqs = 4096;
// int32 fields of an item record
constexpr int kItemInts = 8;
enum ItemField { kItB = 0, kItHg, kItTile, kItKtLo, kItKtHi, kItChunk, kItSplit, kItSlot };  // chunk | nchunks << 16
// int32 header: queue heads [0, 8), item counts [8, 16), then:
constexpr int kHdrCap = 16, kHdrOverflow = 17, kHdrSplits = 18, kHdrSlots = 19, kHdrInts = 64;

struct PrefillPlanLayout {
  int32_t items_cap;  // item records per die
  int32_t split_cap;  // split query tiles (arrival counters)
  int32_t slot_cap;   // softmax-state slots
  int64_t state_floats;  // floats per slot
  int64_t hdr, items, arrive, mailbox, states, timeline, total;  // byte offsets, total bytes
};

__host__ __device__ inline int64_t plan_align(int64_t x) { return (x + 255) & ~(int64_t)255; }

// qp: query positions per tile; nhg: head groups (query heads / heads per tile).
__host__ __device__ inline PrefillPlanLayout prefill_plan_layout(int32_t num_seqs, int32_t max_seqlen_q, int32_t nhg,
                                                                 int32_t qp, int32_t head_dim) {
  PrefillPlanLayout L{};
  const int64_t pairs_per_die = ((int64_t)num_seqs * nhg + kPlanXcds - 1) / kPlanXcds;
  const int64_t tiles_q = ((int64_t)max_seqlen_q + qp - 1) / qp;
  // every piece beyond a query tile's first is at least `cap` key tiles, and
  // cap >= (a die's key tiles) / (kPlanItemsPerCu * kPlanCusPerXcd)
  const int64_t extra = (int64_t)kPlanItemsPerCu * kPlanCusPerXcd;
  L.items_cap = (int32_t)(pairs_per_die * tiles_q + extra + 8);
  L.split_cap = (int32_t)(extra * kPlanXcds);
  L.slot_cap = 2 * L.split_cap;
  L.state_floats = (int64_t)8 * (head_dim / 32 * 16 + 2) * 64;  // 8 waves x (accumulators + m + l) x 64 lanes
  int64_t off = 0;
  L.hdr = off;     off = plan_align(off + kHdrInts * 4);
  L.items = off;   off = plan_align(off + (int64_t)kPlanXcds * L.items_cap * kItemInts * 4);
  L.arrive = off;  off = plan_align(off + (int64_t)L.split_cap * kPlanWaves * 4);
  L.mailbox = off; off = plan_align(off + (int64_t)kPersistWgs * 2 * 4);
  L.states = off;  off = plan_align(off + (int64_t)L.slot_cap * L.state_floats * 4);
#ifdef PKV_PREFILL_TIMELINE
  L.timeline = off; off = plan_align(off + (int64_t)kPersistWgs * kTimelineItems * kTimelineFields * 8);
#endif
  L.total = off;
  return L;
}

struct PrefillPlanArgs {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t num_seqs;
  int32_t nhg;
  int32_t qp;
  int32_t items_cap;
  int32_t split_cap;
  int32_t slot_cap;
  int32_t* hdr;
  int32_t* items;
  int32_t* arrive;
};

hipError_t launch_prefill_plan(const PrefillPlanArgs& p, hipStream_t stream);
// Query positions per tile and head groups of the matrix-core prefill for these heads.
int prefill_tile_positions(int32_t num_q_heads, int32_t num_kv_heads);
int prefill_head_groups(int32_t num_q_heads, int32_t num_kv_heads);

// bf16 matrix-core prefill: one workgroup per query tile (plan_hdr NULL), or the
// persistent kernel over the plan's work lists (after launch_prefill_plan).
hipError_t launch_prefill_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream);

// bf16 matrix-core group pass of shared-prefix decode (same kernel, gathered queries).
hipError_t launch_shared_prefix_mfma(const PrefillArgs& a, int32_t head_dim, hipStream_t stream);
// Members per workgroup of the group pass for this head grouping.
int shared_prefix_members_per_wg(int32_t num_q_heads, int32_t num_kv_heads);
// Workgroups of the group pass per chunk of keys.
int64_t shared_prefix_wgs_per_chunk(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_groups,
                                    int32_t max_group_size);

// Arguments of the fused rotary embedding + cache write.
struct RopeStoreArgs {
  void* q;                       // [num_tokens, num_q_heads, D], rotated in place
  const void* k;                 // [num_tokens, num_kv_heads, D]
  const void* v;                 // [num_tokens, num_kv_heads, D]
  const int32_t* positions;      // [num_tokens]
  void* k_cache;                 // [num_blocks * block_size, num_kv_heads, D]
  void* v_cache;
  const int32_t* slot_mapping;   // [num_tokens], negative = no cache write
  int64_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  double log2_theta;             // pair j turns by position * 2^(-2j/D * log2_theta)
};

hipError_t launch_rope_kv_store(const RopeStoreArgs& a, int32_t dtype, int32_t head_dim, bool interleaved,
                                hipStream_t stream);

// Precondition checks: counter index of each kind of violation (the same
// numbers as pkv_check_flag in pkv.h).
enum CheckCode : int32_t {
  kCheckLength = 0,
  kCheckBlockId = 1,
  kCheckCuSeqlens = 2,
  kCheckSlot = 3,
  kCheckDuplicateSlot = 4,
  kCheckSharedPrefix = 5,
  kCheckGroup = 6,
  kCheckNumFlags = 8,
};

struct CheckArgs {
  const int32_t* block_tables;  // NULL: no table (packed prefill)
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;  // decode and groups; NULL for prefill
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t max_len_q;
  int32_t max_len_k;
  int32_t num_seqs;
  int64_t num_blocks;
  int32_t block_size;
  const int32_t* slot_mapping;
  int64_t num_tokens;
  uint32_t* bitmap;  // one bit per slot, or NULL (no duplicate check)
  const int32_t* shared_lens;
  const int32_t* group_offsets;
  const int32_t* group_seqs;
  int32_t num_groups;
  int32_t num_members;  // entries of group_seqs
  int32_t max_group_size;
  int32_t max_shared_len;
  int32_t* seen;   // [num_seqs] groups naming each sequence
  int32_t* flags;  // [kCheckNumFlags]
};

hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t stream);
hipError_t launch_check_tables(const CheckArgs& a, hipStream_t stream);
hipError_t launch_check_slots(const CheckArgs& a, hipStream_t stream);
hipError_t launch_check_groups(const CheckArgs& a, hipStream_t stream);

// Row-attention instantiation exists for this shape?
bool row_attn_supported(int32_t dtype, int32_t head_dim, int32_t num_q_heads, int32_t num_kv_heads);

}  // namespace pkv
