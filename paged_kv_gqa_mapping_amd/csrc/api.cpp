// C ABI of libpkv.so: argument checks, split choice, and launches on the
// caller's stream.  Declarations and the full contract are in include/pkv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/pkv.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : 4; }

int log2_exact(int32_t x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

// Shape checks common to every call on the cache.
int check_cache_shape(int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                      bool paged) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not PKV_F32 or PKV_BF16", dtype);
  if (num_kv_heads < 1 || num_kv_heads > 64)
    return fail(num_kv_heads < 1 ? PKV_ERR_INVALID_ARG : PKV_ERR_UNSUPPORTED, "num_kv_heads %d outside [1, 64]",
                num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", head_dim);
  if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks %lld < 1", (long long)num_blocks);
  if (paged) {
    const int lb = log2_exact(block_size);
    if (block_size < 8 || block_size > 1024 || lb < 0)
      return fail(PKV_ERR_UNSUPPORTED, "block_size %d is not a power of two in [8, 1024]", block_size);
  }
  return PKV_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "group size %d (num_q_heads / num_kv_heads) is not 1, 2, 4 or 8", G);
  return PKV_OK;
}

int32_t round_up(int64_t x, int32_t m) { return (int32_t)(((x + m - 1) / m) * m); }

// Split length for decode (tokens): a power of two, the smallest that keeps
// the grid near 4096 waves (16 per CU) so that every CU has work, but at
// least 512 tokens (256 when the longest context is at most 1024) so that a
// wave's fixed costs (first loads, partial-state write) stay small next to
// its streaming time.  A context of at most 256 tokens is one split.
int32_t auto_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  if (max_context_len <= 256) return round_up(std::max(max_context_len, 1), 64);
  const int64_t base = (int64_t)num_seqs * std::max(1, num_kv_heads / 8);
  const int64_t want_splits = std::max<int64_t>(1, (4096 + base - 1) / base);
  const int64_t need = (max_context_len + want_splits - 1) / want_splits;
  int32_t split = max_context_len <= 1024 ? 256 : 512;
  while (split < need && split < max_context_len) split *= 2;
  return split;
}

// Token-balanced decode (split_tokens = PKV_SPLIT_BALANCED): the batch's
// steps (U tokens each), sequence after sequence, are cut into kBalancePieces
// nearly equal ranges (row_attn.hpp), one wave each per group of KV heads, so
// that the waves of a launch finish together whatever the mix of context
// lengths; a multiple of the 256 compute units, so that each unit holds as
// many waves.
#ifndef PKV_BALANCE_PIECES
#define PKV_BALANCE_PIECES 1024
#endif
constexpr int32_t kBalancePieces = PKV_BALANCE_PIECES;
// State rows [W + B, Hq] (slot w + b for the part of sequence b in wave w's
// range), then with shared prefixes [B, Hq, C] for the group pass's chunks;
// D floats each in ws_o and 2 in ws_ml, then [B, 2] ints (first slot, count).
int64_t balanced_rows(int32_t num_seqs, int32_t num_q_heads, int32_t prefix_states) {
  return ((int64_t)kBalancePieces + num_seqs) * num_q_heads + (int64_t)num_seqs * num_q_heads * prefix_states;
}
int64_t balanced_state_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t prefix_states = 0) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return balanced_rows(num_seqs, num_q_heads, prefix_states) * (head_dim + 2) * (int64_t)sizeof(float) +
         (int64_t)num_seqs * 2 * (int64_t)sizeof(int32_t);
}
// The library's choice for split_tokens = 0: token-balanced ranges for any
// context longer than 256 tokens (equal work per wave whatever the mix of
// lengths; measured faster than the fixed split on every shape tried), and
// one split per sequence for contexts of at most 256 tokens (auto_split).
bool auto_balanced(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  return num_seqs >= 1 && num_kv_heads >= 1 && max_context_len > 256;
}

struct DecodeCall {
  pkv::RowAttnArgs args;
  int32_t dtype;
  int32_t head_dim;
  bool empty;
};

// Launch plan of a decode call: split length and count, and for shared-prefix
// decode the group pass's chunk length and count (prefix states per pair).
struct DecodePlan {
  int32_t split = 0;
  int32_t S = 1;      // split states per pair (grid splits)
  int32_t chunk = 0;  // keys per group-pass state
  int32_t C = 0;      // group-pass states per pair
  bool balanced = false;  // own keys in token-balanced ranges instead of splits
};

// Shared-prefix plan.  The split pass only covers each sequence's own keys,
// so its split comes from the longest of those (max_own_len).  The group pass
// takes chunks of at least 256 keys (4 tiles), doubled while its grid would
// need more than one round of 512 workgroups (2 per CU): a longer chunk then
// costs no time in that pass and halves the states the merge reads.
DecodePlan cascade_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                        int32_t max_own_len, int32_t split_tokens, int32_t num_groups, int32_t max_group_size,
                        int32_t max_shared_len) {
  DecodePlan p;
  const int32_t own = (max_own_len > 0 && max_own_len < max_context_len) ? max_own_len : max_context_len;
  p.split = split_tokens;
  // token-balanced ranges when asked for, or when the own keys could give each
  // of the kBalancePieces waves 256 of them; fewer own keys keep the fine
  // splits below, which run more (shorter) waves
  p.balanced = split_tokens == PKV_SPLIT_BALANCED ||
               (split_tokens == 0 && own > 256 &&
                (int64_t)std::max(num_seqs, 1) * own >= (int64_t)kBalancePieces * 256);
  if (p.balanced) {
    p.split = 0;
    p.S = kBalancePieces;
  } else if (!p.split) {
    // Own keys are often few (a short suffix behind a long shared prompt), and the
    // plain rule's 256/512-token floor would then leave a small grid of long
    // waves; splits down to 64 keys keep about 2048 waves in flight.  Long own
    // keys keep the plain rule.
    const int64_t base = (int64_t)std::max(num_seqs, 1) * std::max(1, num_kv_heads / 8);
    int32_t fine = 64;
    while (fine < own && base * ((own + fine - 1) / fine) > 2048) fine *= 2;
    p.split = std::min(fine, auto_split(std::max(num_seqs, 1), std::max(num_kv_heads, 1), own));
  }
  if (!p.balanced) p.S = std::max(1, (own + p.split - 1) / p.split);
  if (num_groups > 0 && max_shared_len > 0) {
    // chunks of the shared prefix: from 256 keys, doubled while the group pass
    // would have more workgroups than the 256 CUs hold at once (one each: the
    // pass stages its K/V tiles in 96 KB of LDS); fewer, longer chunks also
    // leave fewer states per member for the merge
    const int64_t wgs = pkv::shared_prefix_wgs_per_chunk(num_q_heads, num_kv_heads, num_groups, max_group_size);
    p.chunk = 256;
    while (p.chunk < max_shared_len && wgs * ((max_shared_len + p.chunk - 1) / p.chunk) > 256) p.chunk *= 2;
    p.C = (max_shared_len + p.chunk - 1) / p.chunk;
  }
  return p;
}

// Workspace of S split states plus C prefix states per (sequence, query head); none when a
// single state per pair is written straight to the output.
int64_t state_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int64_t S, int64_t C) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || S <= 0) return 0;
  if (S + C <= 1) return 0;
  return (int64_t)num_seqs * num_q_heads * (S + C) * (head_dim + 2) * (int64_t)sizeof(float);
}

int prepare_decode(DecodeCall& call, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                   int32_t max_context_len, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                   int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                   const DecodePlan* plan = nullptr) {
  call.empty = false;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  int st = check_cache_shape(num_kv_heads, head_dim, num_blocks, block_size, dtype, true);
  if (st) return st;
  st = check_heads(num_q_heads, num_kv_heads);
  if (st) return st;
  if (num_seqs == 0) {
    call.empty = true;
    return PKV_OK;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer among q, k_cache, v_cache, block_tables, context_lens, out");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len %d outside [0, max_blocks_per_seq * block_size = %lld]",
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (split_tokens != PKV_SPLIT_BALANCED && (split_tokens < 0 || split_tokens % 64))
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d is not 0, PKV_SPLIT_BALANCED or a positive multiple of 64",
                split_tokens);
  const bool balanced = plan ? plan->balanced
                             : (split_tokens == PKV_SPLIT_BALANCED ||
                                (split_tokens == 0 && auto_balanced(num_seqs, num_kv_heads, max_context_len)));
  const int32_t split = balanced ? 0
                        : plan   ? plan->split
                        : split_tokens ? split_tokens
                                       : auto_split(num_seqs, num_kv_heads, max_context_len);
  const int32_t S = balanced ? kBalancePieces : plan ? plan->S : std::max(1, (max_context_len + split - 1) / split);
  const int32_t prefix_states = plan ? plan->C : 0;
  const int64_t need = balanced ? balanced_state_bytes(num_seqs, num_q_heads, head_dim, prefix_states)
                                : state_bytes(num_seqs, num_q_heads, head_dim, S, prefix_states);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "decode workspace of %lld bytes needed, %lld given%s", (long long)need,
                (long long)workspace_bytes, workspace ? "" : " (NULL)");
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u))
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if ((int64_t)(balanced ? 1 : num_seqs) * (num_kv_heads) * S > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "grid too large: reduce num_seqs or raise split_tokens");

  pkv::RowAttnArgs& a = call.args;
  a = pkv::RowAttnArgs{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.ws_o = need > 0 ? static_cast<float*>(workspace) : nullptr;
  const int64_t state_rows = balanced ? balanced_rows(num_seqs, num_q_heads, prefix_states)
                                      : (int64_t)num_seqs * num_q_heads * (S + prefix_states);
  a.ws_ml = need > 0 ? a.ws_o + state_rows * head_dim : nullptr;
  if (balanced) {
    a.balance_pieces = S;
    a.piece_meta = reinterpret_cast<int32_t*>(a.ws_ml + state_rows * 2);
    a.prefix_slot0 = ((int64_t)S + num_seqs) * num_q_heads;
    a.prefix_states = prefix_states;
  }
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.log2_block_size = log2_exact(block_size);
  a.split_tokens = split;
  a.num_splits = S;
  a.ws_stride = balanced ? 1 : S + prefix_states;
  a.prefix_chunk = plan ? plan->chunk : 0;
  call.dtype = dtype;
  call.head_dim = head_dim;
  if (!pkv::row_attn_supported(dtype, head_dim, num_q_heads, num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "no decode kernel for dtype %d, head_dim %d, %d/%d heads", dtype, head_dim,
                num_q_heads, num_kv_heads);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
  }
  return "unknown pkv status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_kv_store(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                 int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                 int32_t dtype, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  int st = check_cache_shape(num_kv_heads, head_dim, num_blocks, block_size, dtype, true);
  if (st) return st;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer among k, v, k_cache, v_cache, slot_mapping");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
  if (num_tokens > 0x7fffffffLL * 4) return fail(PKV_ERR_UNSUPPORTED, "num_tokens %lld too large", (long long)num_tokens);
  const int32_t row_bytes = num_kv_heads * head_dim * elt_bytes(dtype);
  return hip_status(pkv::launch_kv_store(k, v, k_cache, v_cache, slot_mapping, num_tokens, row_bytes,
                                         static_cast<hipStream_t>(stream)),
                    "kv_store launch");
}

int pkv_rope_kv_store(void* q, const void* k, const void* v, const int32_t* positions, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks, int32_t block_size, double rope_theta,
                      int32_t interleaved, int32_t dtype, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  int st = check_cache_shape(num_kv_heads, head_dim, num_blocks, block_size, dtype, true);
  if (st) return st;
  if (num_q_heads < 1 || num_q_heads > 1024)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d outside [1, 1024]", num_q_heads);
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta))
    return fail(PKV_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (interleaved != 0 && interleaved != 1) return fail(PKV_ERR_INVALID_ARG, "interleaved %d is not 0 or 1", interleaved);
  if (num_tokens == 0) return PKV_OK;
  if (!q || !k || !v || !positions || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer among q, k, v, positions, k_cache, v_cache, slot_mapping");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "q, k, v, k_cache and v_cache must be 16-byte aligned");
  if (num_tokens > 0x7fffffffLL) return fail(PKV_ERR_UNSUPPORTED, "num_tokens %lld too large", (long long)num_tokens);
  pkv::RopeStoreArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.log2_theta = std::log2(rope_theta);
  return hip_status(pkv::launch_rope_kv_store(a, dtype, head_dim, interleaved != 0, static_cast<hipStream_t>(stream)),
                    "rope_kv_store launch");
}

int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t block_size, int32_t dtype) {
  (void)num_q_heads;
  (void)head_dim;
  (void)block_size;
  (void)dtype;
  if (auto_balanced(num_seqs, num_kv_heads, max_context_len)) return PKV_SPLIT_BALANCED;
  return auto_split(std::max(num_seqs, 1), std::max(num_kv_heads, 1), std::max(max_context_len, 0));
}

int64_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                   int32_t split_tokens) {
  if (split_tokens == PKV_SPLIT_BALANCED) return balanced_state_bytes(num_seqs, num_q_heads, head_dim);
  if (max_context_len <= 0 || split_tokens <= 0) return 0;
  const int64_t S = (max_context_len + (int64_t)split_tokens - 1) / split_tokens;
  return state_bytes(num_seqs, num_q_heads, head_dim, S, 0);
}

int64_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t max_own_len, int32_t split_tokens,
                                    int32_t num_groups, int32_t max_group_size, int32_t max_shared_len) {
  if (max_context_len <= 0 || (split_tokens < 0 && split_tokens != PKV_SPLIT_BALANCED) || max_shared_len < 0 ||
      num_groups < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return 0;
  const bool cascade = num_groups > 0 && max_shared_len > 0;
  const DecodePlan p = cascade_plan(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                    cascade ? max_own_len : 0, split_tokens, cascade ? num_groups : 0,
                                    max_group_size, cascade ? max_shared_len : 0);
  return p.balanced ? balanced_state_bytes(num_seqs, num_q_heads, head_dim, p.C)
                    : state_bytes(num_seqs, num_q_heads, head_dim, p.S, p.C);
}

#define PKV_DECODE_ARGS                                                                                        \
  const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,                      \
      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len, float scale, void *out, \
      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,      \
      int32_t block_size, int32_t dtype, int32_t split_tokens, void *workspace, int64_t workspace_bytes,      \
      void *stream
#define PKV_DECODE_FWD                                                                                        \
  q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, out, num_seqs, \
      num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, dtype, split_tokens, workspace, workspace_bytes

int pkv_paged_decode_split(PKV_DECODE_ARGS) {
  DecodeCall call;
  int st = prepare_decode(call, PKV_DECODE_FWD);
  if (st || call.empty) return st;
  return hip_status(pkv::launch_row_attn(call.args, call.dtype, call.head_dim, false, static_cast<hipStream_t>(stream)),
                    "decode split launch");
}

int pkv_paged_decode_reduce(PKV_DECODE_ARGS) {
  DecodeCall call;
  int st = prepare_decode(call, PKV_DECODE_FWD);
  if (st || call.empty) return st;
  if (call.args.num_splits <= 1) return PKV_OK;
  return hip_status(pkv::launch_decode_reduce(call.args, call.dtype, call.head_dim, static_cast<hipStream_t>(stream)),
                    "decode reduce launch");
}

int pkv_paged_decode_attn(PKV_DECODE_ARGS) {
  DecodeCall call;
  int st = prepare_decode(call, PKV_DECODE_FWD);
  if (st || call.empty) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pkv::launch_row_attn(call.args, call.dtype, call.head_dim, false, s), "decode split launch");
  if (st || call.args.num_splits <= 1) return st;
  return hip_status(pkv::launch_decode_reduce(call.args, call.dtype, call.head_dim, s), "decode reduce launch");
}

// ---------------------------------------------------------------- allocation-free decode
//
// pkv_paged_decode_attn_noalloc keeps the split-K states in `scratch`, a
// file-scope device array: each GPU the library runs on holds one copy of it
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in): the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and every use goes through it.
}  // extern "C"

namespace {
constexpr int64_t kScratchBytes = 64ll << 20;  // the limit stated in pkv.h
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of each GPU's copy (nullptr until its first call)
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
// This device's copy of the scratch array; the stream must belong to the current device.
int scratch_of_current_device(void* stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(PKV_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the first %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PKV_OK;
}
}  // namespace

extern "C" {

int64_t pkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pkv_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                                  float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                                  int32_t split_tokens, void* stream) {
  void* ws = nullptr;
  int st = scratch_of_current_device(stream, &ws);
  if (st) return st;
  DecodeCall call;
  st = prepare_decode(call, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                      out, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, dtype, split_tokens,
                      ws, kScratchBytes);
  if (st == PKV_ERR_WORKSPACE) {
    // (the sizes were valid: the workspace is checked after them)
    const int32_t split = split_tokens ? split_tokens
                                       : pkv_decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                                 max_context_len, block_size, dtype);
    return fail(PKV_ERR_WORKSPACE,
                "the split states of this call need %lld bytes, above the %lld-byte scratch of the allocation-free "
                "entry point: raise split_tokens or use pkv_paged_decode_attn with a workspace",
                (long long)pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, split),
                (long long)kScratchBytes);
  }
  if (st || call.empty) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pkv::launch_row_attn(call.args, call.dtype, call.head_dim, false, s), "decode split launch");
  if (st || call.args.num_splits <= 1) return st;
  return hip_status(pkv::launch_decode_reduce(call.args, call.dtype, call.head_dim, s), "decode reduce launch");
}

int pkv_paged_decode_store_attn(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                int32_t dtype, int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  DecodeCall call;
  int st = prepare_decode(call, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                          scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, dtype,
                          split_tokens, workspace, workspace_bytes);
  if (st || call.empty) return st;
  if (!k || !v) return fail(PKV_ERR_INVALID_ARG, "null k or v (the new tokens)");
  if (!aligned16(k) || !aligned16(v)) return fail(PKV_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  call.args.k_new = k;
  call.args.v_new = v;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pkv::launch_row_attn(call.args, call.dtype, call.head_dim, false, s), "decode split launch");
  if (st || call.args.num_splits <= 1) return st;
  return hip_status(pkv::launch_decode_reduce(call.args, call.dtype, call.head_dim, s), "decode reduce launch");
}

int pkv_cascade_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                            const int32_t* shared_lens, const int32_t* group_offsets, const int32_t* group_seqs,
                            int32_t num_groups, int32_t max_group_size, int32_t max_shared_len, int32_t max_own_len,
                            float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                            int32_t split_tokens, void* workspace, int64_t workspace_bytes, void* stream) {
  if (num_groups < 0 || max_group_size < 0 || max_shared_len < 0 || max_own_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative group count, group size, shared length or own length");
  const bool cascade = num_groups > 0 && max_shared_len > 0;
  if (cascade) {
    if (dtype != PKV_BF16)
      return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode needs bf16 (its group pass runs on the matrix cores)");
    if (!shared_lens || !group_offsets || !group_seqs)
      return fail(PKV_ERR_INVALID_ARG, "null pointer among shared_lens, group_offsets, group_seqs");
    if (max_group_size < 1) return fail(PKV_ERR_INVALID_ARG, "max_group_size %d < 1", max_group_size);
    if (max_shared_len >= max_context_len)
      return fail(PKV_ERR_INVALID_ARG, "max_shared_len %d must be below max_context_len %d", max_shared_len,
                  max_context_len);
    if (max_shared_len % block_size)
      return fail(PKV_ERR_INVALID_ARG, "max_shared_len %d is not a whole number of blocks of %d", max_shared_len,
                  block_size);
    // the group pass takes the max of raw scores before scaling and masks keys
    // past a chunk's end with -inf, both of which need a positive scale
    if (!(scale > 0.f) || !std::isfinite(scale))
      return fail(PKV_ERR_INVALID_ARG, "shared-prefix decode needs a finite scale > 0 (got %g)", (double)scale);
  }
  if (split_tokens != PKV_SPLIT_BALANCED && (split_tokens < 0 || split_tokens % 64))
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d is not 0, PKV_SPLIT_BALANCED or a positive multiple of 64",
                split_tokens);
  int st = check_heads(num_q_heads, num_kv_heads);
  if (st) return st;
  const DecodePlan plan = cascade_plan(num_seqs, num_q_heads, num_kv_heads, std::max(max_context_len, 1),
                                       cascade ? max_own_len : 0, split_tokens, cascade ? num_groups : 0,
                                       max_group_size, cascade ? max_shared_len : 0);
  DecodeCall call;
  st = prepare_decode(call, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                      scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, dtype,
                      split_tokens, workspace, workspace_bytes, &plan);
  if (st || call.empty) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pkv::RowAttnArgs& r = call.args;
  if (cascade) {
    pkv::PrefillArgs g{};
    g.q = q;
    g.k = k_cache;
    g.v = v_cache;
    g.block_tables = block_tables;
    g.scale_log2 = r.scale_log2;
    g.num_seqs = num_seqs;
    g.num_q_heads = num_q_heads;
    g.num_kv_heads = num_kv_heads;
    g.max_blocks_per_seq = max_blocks_per_seq;
    g.log2_block_size = r.log2_block_size;
    g.group_offsets = group_offsets;
    g.group_seqs = group_seqs;
    g.shared_lens = shared_lens;
    if (r.balance_pieces > 0) {
      // the chunk states' own region: pair p's chunk c at row p * C + c of it
      g.ws_o = r.ws_o + r.prefix_slot0 * head_dim;
      g.ws_ml = r.ws_ml + r.prefix_slot0 * 2;
      g.ws_stride = plan.C;
      g.slot0 = 0;
    } else {
      g.ws_o = r.ws_o;
      g.ws_ml = r.ws_ml;
      g.ws_stride = r.ws_stride;
      g.slot0 = r.num_splits;
    }
    g.chunk_tokens = plan.chunk;
    g.num_groups = num_groups;
    g.num_chunks = plan.C;
    const int per_wg = pkv::shared_prefix_members_per_wg(num_q_heads, num_kv_heads);
    g.member_tiles = (max_group_size + per_wg - 1) / per_wg;
    st = hip_status(pkv::launch_shared_prefix_mfma(g, head_dim, s), "shared-prefix group pass launch");
    if (st) return st;
    r.kv_start = shared_lens;
  }
  st = hip_status(pkv::launch_row_attn(r, call.dtype, call.head_dim, false, s), "decode split launch");
  if (st || (!cascade && r.num_splits <= 1)) return st;
  return hip_status(pkv::launch_decode_reduce(r, call.dtype, call.head_dim, s), "decode reduce launch");
}

int64_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t max_seqlen_q, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t dtype) {
  if (dtype != PKV_BF16 || num_seqs <= 0 || max_seqlen_q <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads || (head_dim != 64 && head_dim != 128))
    return 0;
  return pkv::prefill_plan_layout(num_seqs, max_seqlen_q, pkv::prefill_head_groups(num_q_heads, num_kv_heads),
                                  pkv::prefill_tile_positions(num_q_heads, num_kv_heads), head_dim)
      .total;
}

int pkv_paged_prefill_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           void* out, float scale, int32_t num_seqs, int64_t total_q, int32_t max_seqlen_q,
                           int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int64_t num_blocks, int32_t block_size, int32_t dtype, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size");
  const bool paged = block_tables != nullptr;
  int st = check_cache_shape(num_kv_heads, head_dim, num_blocks, block_size, dtype, paged);
  if (st) return st;
  st = check_heads(num_q_heads, num_kv_heads);
  if (st) return st;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer among q, k, v, cu_seqlens_q, cu_seqlens_k, out");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PKV_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (max_seqlen_q > max_seqlen_k)
    return fail(PKV_ERR_INVALID_ARG, "max_seqlen_q %d > max_seqlen_k %d", max_seqlen_q, max_seqlen_k);
  if (paged && (max_blocks_per_seq < 1 || (int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * block_size))
    return fail(PKV_ERR_INVALID_ARG, "max_seqlen_k %d exceeds max_blocks_per_seq %d * block_size %d", max_seqlen_k,
                max_blocks_per_seq, block_size);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PKV_BF16) {
    pkv::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.block_tables = block_tables;
    a.cu_seqlens_q = cu_seqlens_q;
    a.cu_seqlens_k = cu_seqlens_k;
    a.out = out;
    a.scale_log2 = sc * 1.4426950408889634f;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.log2_block_size = paged ? log2_exact(block_size) : 0;
    a.max_seqlen_q = max_seqlen_q;
    if (workspace && num_seqs <= pkv::kPlanMaxSeqs) {
      // persistent kernel over the work lists the plan kernel writes into the workspace
      const int nhg = pkv::prefill_head_groups(num_q_heads, num_kv_heads);
      const int qp = pkv::prefill_tile_positions(num_q_heads, num_kv_heads);
      const pkv::PrefillPlanLayout L = pkv::prefill_plan_layout(num_seqs, max_seqlen_q, nhg, qp, head_dim);
      if (workspace_bytes < L.total)
        return fail(PKV_ERR_WORKSPACE, "prefill workspace of %lld bytes needed, %lld given", (long long)L.total,
                    (long long)workspace_bytes);
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PKV_ERR_INVALID_ARG, "prefill workspace must be 256-byte aligned");
      uint8_t* w = static_cast<uint8_t*>(workspace);
      pkv::PrefillPlanArgs p{};
      p.cu_seqlens_q = cu_seqlens_q;
      p.cu_seqlens_k = cu_seqlens_k;
      p.num_seqs = num_seqs;
      p.nhg = nhg;
      p.qp = qp;
      p.items_cap = L.items_cap;
      p.split_cap = L.split_cap;
      p.slot_cap = L.slot_cap;
      p.hdr = reinterpret_cast<int32_t*>(w + L.hdr);
      p.items = reinterpret_cast<int32_t*>(w + L.items);
      p.arrive = reinterpret_cast<int32_t*>(w + L.arrive);
      int st2 = hip_status(pkv::launch_prefill_plan(p, s), "prefill plan launch");
      if (st2) return st2;
      a.plan_hdr = p.hdr;
      a.plan_queue = p.hdr;
      a.plan_items = p.items;
      a.plan_arrive = p.arrive;
      a.plan_mailbox = reinterpret_cast<int32_t*>(w + L.mailbox);
      a.plan_states = reinterpret_cast<float*>(w + L.states);
#ifdef PKV_PREFILL_TIMELINE
      a.timeline = reinterpret_cast<long long*>(w + L.timeline);
#endif
      a.items_cap = L.items_cap;
    }
    return hip_status(pkv::launch_prefill_mfma(a, head_dim, s), "prefill launch");
  }
  if (!pkv::row_attn_supported(dtype, head_dim, num_q_heads, num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "no prefill kernel for dtype %d, head_dim %d, %d/%d heads", dtype, head_dim,
                num_q_heads, num_kv_heads);
  pkv::RowAttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_tables = block_tables;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.out = out;
  a.scale_log2 = sc * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.log2_block_size = paged ? log2_exact(block_size) : 0;
  a.max_rows = max_seqlen_q;
  return hip_status(pkv::launch_row_attn(a, dtype, head_dim, true, s), "prefill launch");
}

// ---------------------------------------------------------------- precondition checks

static_assert(pkv::kCheckLength == PKV_CHECK_LENGTH && pkv::kCheckBlockId == PKV_CHECK_BLOCK_ID &&
                  pkv::kCheckCuSeqlens == PKV_CHECK_CU_SEQLENS && pkv::kCheckSlot == PKV_CHECK_SLOT &&
                  pkv::kCheckDuplicateSlot == PKV_CHECK_DUPLICATE_SLOT &&
                  pkv::kCheckSharedPrefix == PKV_CHECK_SHARED_PREFIX && pkv::kCheckGroup == PKV_CHECK_GROUP &&
                  pkv::kCheckNumFlags == PKV_CHECK_NUM_FLAGS,
              "check codes of the kernels and of the header differ");

int pkv_check_decode_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs, int64_t num_blocks, int32_t block_size,
                            int32_t* flags, void* stream) {
  if (!flags) return fail(PKV_ERR_INVALID_ARG, "flags is NULL");
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "negative or empty size");
  if (num_seqs > 0 && (!block_tables || !context_lens))
    return fail(PKV_ERR_INVALID_ARG, "null block_tables or context_lens");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(pkv::launch_zero(flags, PKV_CHECK_NUM_FLAGS, s), "check launch");
  if (st) return st;
  pkv::CheckArgs a{};
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_len_k = max_context_len;
  a.num_seqs = num_seqs;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.flags = flags;
  return hip_status(pkv::launch_check_tables(a, s), "check launch");
}

int pkv_check_prefill_inputs(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int64_t num_blocks, int32_t block_size, int32_t* flags, void* stream) {
  if (!flags) return fail(PKV_ERR_INVALID_ARG, "flags is NULL");
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_blocks < 1 || block_size < 1 ||
      (block_tables && max_blocks_per_seq < 1))
    return fail(PKV_ERR_INVALID_ARG, "negative or empty size");
  if (num_seqs > 0 && (!cu_seqlens_q || !cu_seqlens_k))
    return fail(PKV_ERR_INVALID_ARG, "null cu_seqlens_q or cu_seqlens_k");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(pkv::launch_zero(flags, PKV_CHECK_NUM_FLAGS, s), "check launch");
  if (st) return st;
  pkv::CheckArgs a{};
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.max_len_q = max_seqlen_q;
  a.max_len_k = max_seqlen_k;
  a.num_seqs = num_seqs;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.flags = flags;
  return hip_status(pkv::launch_check_tables(a, s), "check launch");
}

int pkv_check_slots(const int32_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                    uint32_t* bitmap, int32_t* flags, void* stream) {
  if (!flags) return fail(PKV_ERR_INVALID_ARG, "flags is NULL");
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1) return fail(PKV_ERR_INVALID_ARG, "negative or empty size");
  if (num_tokens > 0 && !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "slot_mapping is NULL");
  if (num_blocks * block_size > 0x7fffffffLL) return fail(PKV_ERR_UNSUPPORTED, "pool larger than int32 slots");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(pkv::launch_zero(flags, PKV_CHECK_NUM_FLAGS, s), "check launch");
  if (st) return st;
  if (bitmap) {
    st = hip_status(pkv::launch_zero(reinterpret_cast<int32_t*>(bitmap), (num_blocks * block_size + 31) / 32, s),
                    "check launch");
    if (st) return st;
  }
  pkv::CheckArgs a{};
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.bitmap = bitmap;
  a.flags = flags;
  return hip_status(pkv::launch_check_slots(a, s), "check launch");
}

int pkv_check_cascade_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             const int32_t* shared_lens, const int32_t* group_offsets, const int32_t* group_seqs,
                             int32_t num_groups, int32_t num_members, int32_t num_seqs, int32_t max_group_size,
                             int32_t max_shared_len, int32_t block_size, int32_t* seen, int32_t* flags, void* stream) {
  if (!flags || !seen) return fail(PKV_ERR_INVALID_ARG, "flags or seen is NULL");
  if (num_groups < 0 || num_members < 0 || num_seqs < 0 || max_group_size < 0 || max_shared_len < 0 ||
      max_blocks_per_seq < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "negative or empty size");
  if (num_seqs > 0 && (!block_tables || !context_lens || !shared_lens))
    return fail(PKV_ERR_INVALID_ARG, "null block_tables, context_lens or shared_lens");
  if (num_groups > 0 && (!group_offsets || (num_members > 0 && !group_seqs)))
    return fail(PKV_ERR_INVALID_ARG, "null group_offsets or group_seqs");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(pkv::launch_zero(flags, PKV_CHECK_NUM_FLAGS, s), "check launch");
  if (!st) st = hip_status(pkv::launch_zero(seen, num_seqs, s), "check launch");
  if (st) return st;
  pkv::CheckArgs a{};
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.block_size = block_size;
  a.shared_lens = shared_lens;
  a.group_offsets = group_offsets;
  a.group_seqs = group_seqs;
  a.num_groups = num_groups;
  a.num_members = num_members;
  a.max_group_size = max_group_size;
  a.max_shared_len = max_shared_len;
  a.seen = seen;
  a.flags = flags;
  return hip_status(pkv::launch_check_groups(a, s), "check launch");
}

int pkv_paged_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_k,
                     void* k_out, void* v_out, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                     int32_t block_size, int32_t dtype, void* stream) {
  if (num_seqs < 0 || max_seqlen_k < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  int st = check_cache_shape(num_kv_heads, head_dim, num_blocks, block_size, dtype, true);
  if (st) return st;
  if (num_seqs == 0 || max_seqlen_k == 0) return PKV_OK;
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "gather handles at most 65535 sequences per call");
  if (!k_cache || !v_cache || !block_tables || !cu_seqlens_k || !k_out || !v_out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
    return fail(PKV_ERR_INVALID_ARG, "caches and outputs must be 16-byte aligned");
  if (max_blocks_per_seq < 1 || (int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_seqlen_k %d exceeds max_blocks_per_seq %d * block_size %d", max_seqlen_k,
                max_blocks_per_seq, block_size);
  const int32_t row_bytes = num_kv_heads * head_dim * elt_bytes(dtype);
  return hip_status(pkv::launch_gather(k_cache, v_cache, block_tables, max_blocks_per_seq, cu_seqlens_k, num_seqs,
                                       max_seqlen_k, k_out, v_out, row_bytes, log2_exact(block_size),
                                       static_cast<hipStream_t>(stream)),
                    "gather launch");
}

}  // extern "C"
