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
};

// bf16 matrix-core prefill.
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
