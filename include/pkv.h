/*
 * pkv.h -- C ABI of the paged-KV GQA attention library (libpkv.so, gfx950).
 *
 * Three operations of a block-paged inference engine's attention layer, as
 * the nano-vLLM pages describe them: the KV-cache write through a slot
 * mapping, decode attention over the paged cache, and causal varlen prefill
 * attention ("Nano-vLLM Architecture and Performance", section
 * "FlashAttention Integration": prefill and decode attention run through one
 * attention library and a separate store kernel puts each new token's K/V
 * into its cache block; "Project overview and the four-layer architecture",
 * section "Lifecycle of one request", step 4: the new K/V are stored first and
 * attention runs afterwards).
 *
 * Conventions for every call
 * --------------------------
 * - Every pointer argument is a DEVICE pointer unless stated otherwise.  The
 *   caller allocates, owns and frees every buffer; the library never
 *   allocates device memory and keeps no state between calls.
 * - Every call is asynchronous: it enqueues work on `stream` (a hipStream_t
 *   passed as void*, NULL = the default stream) and returns without
 *   synchronizing.  Calls are reentrant and thread-safe.
 * - Element types: `dtype` is PKV_F32 (float) or PKV_BF16 (bfloat16 bit
 *   patterns).  Outputs have the input dtype.  All metadata is int32; element
 *   offsets are computed in 64 bits.
 * - KV cache layout (a reading; the pages print none):
 *       k_cache, v_cache: [num_blocks, block_size, num_kv_heads, head_dim],
 *       row-major, head_dim contiguous, 16-byte aligned.
 *   The token at absolute position p of sequence b lives in physical block
 *   block_tables[b * max_blocks_per_seq + p / block_size], row p % block_size;
 *   its slot is block * block_size + row.
 * - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads) (X-Ray
 *   panel of the nano-vllm README: 32 query heads over 8 KV heads, four per group).
 * - Supported shapes: head_dim 64 or 128; block_size a power of two in
 *   [8, 1024]; num_q_heads / num_kv_heads in {1, 2, 4, 8}; 1 <= num_kv_heads <= 64.
 *   Other shapes return PKV_ERR_UNSUPPORTED.
 * - Errors: the return value is PKV_OK (0) or a negative pkv_status.  Argument
 *   errors are detected on the host before anything is enqueued.  A failed
 *   launch returns PKV_ERR_HIP.  pkv_last_error() gives a thread-local text
 *   for the last non-OK return.  Device-side preconditions (block ids in
 *   [0, num_blocks), distinct slots, 0 <= context_lens <= max_context_len,
 *   cu_seqlens non-decreasing with Lq <= Lk) are the caller's to keep and are
 *   not checked on the device; breaking them gives undefined results.
 * - Zero sizes (num_tokens == 0, num_seqs == 0) return PKV_OK without a launch.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent sizes */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, block size, group size, dtype */
  PKV_ERR_WORKSPACE = -3,   /* decode workspace missing or too small */
  PKV_ERR_HIP = -4,         /* the HIP runtime reported an error (text in pkv_last_error) */
  PKV_ERR_OUT_OF_BLOCKS = -5 /* block manager: not enough free blocks (nothing was changed) */
} pkv_status;

/* Library version: major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/* Text of a status code (static storage). */
const char* pkv_status_string(int status);

/* Thread-local description of the last non-OK return on this thread. */
const char* pkv_last_error(void);

/*
 * kv_store -- write the K and V rows of num_tokens new tokens into the paged
 * caches (the store kernel of "Nano-vLLM Architecture and Performance",
 * section "FlashAttention Integration"; ModelRunner builds the slot_mapping,
 * section "How It Works End-to-End").
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim], contiguous, read only.
 *   k_cache,
 *   v_cache       [num_blocks, block_size, num_kv_heads, head_dim], written.
 *   slot_mapping  [num_tokens] int32.  Token i goes to slot slot_mapping[i]
 *                 (block = slot / block_size, row = slot % block_size).  A
 *                 negative slot skips the token.  Non-negative slots must be
 *                 distinct and < num_blocks * block_size.
 *
 * A pure copy of the stored bits: the caches change only at the named slots.
 */
int pkv_kv_store(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                 int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                 int32_t block_size, int32_t dtype, void* stream);

/*
 * rope_kv_store -- rotary position embedding of q and k, fused with the cache
 * write of the rotated k and of v.  The pages list a rotary embedding layer
 * that runs before attention ("Nano-vLLM Architecture and Performance",
 * project layout, layers/rotary_embedding.py) and a per-token positions
 * array built by the model runner (same page, section "How It Works
 * End-to-End"); they print no formula.  The rotation is the RoFormer one:
 * pair j of every head of token i turns by the angle
 * positions[i] * rope_theta^(-2j / head_dim), i.e. (x, y) becomes
 * (x cos t - y sin t, x sin t + y cos t).
 *
 *   q             [num_tokens, num_q_heads, head_dim], rotated IN PLACE.
 *   k, v          [num_tokens, num_kv_heads, head_dim], read only.
 *   positions     [num_tokens] int32, the token's position in its sequence.
 *   k_cache,
 *   v_cache       [num_blocks, block_size, num_kv_heads, head_dim]; the rotated
 *                 k row and the v row of token i are written at slot
 *                 slot_mapping[i], exactly where pkv_kv_store puts them.  A
 *                 negative slot skips the cache write (q is still rotated).
 *   rope_theta    > 1, the base of the pair frequencies (model constant).
 *   interleaved   0: pair j is (j, j + head_dim/2) ("rotate-half");
 *                 1: pair j is (2j, 2j + 1).
 *
 * Arithmetic: angles are reduced modulo 2 pi in fp64, (cos, sin) and the
 * products are fp32, results rounded to nearest even to the storage dtype,
 * so each output is within one unit in the last place of the exact rotation.
 * v moves bit-exact.  Same preconditions on slots as pkv_kv_store.
 */
int pkv_rope_kv_store(void* q, const void* k, const void* v, const int32_t* positions, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks, int32_t block_size, double rope_theta,
                      int32_t interleaved, int32_t dtype, void* stream);

/*
 * Decode attention, split-K.  Sequence b's single query q[b] attends all
 * context_lens[b] tokens of its context (the token just stored included),
 * read through row b of block_tables: out = softmax(scale * q K^T) V per
 * query head (decode produces a single token per sequence each step and is
 * bound by memory traffic: "Project overview and the four-layer
 * architecture", section "Lifecycle of one request").
 *
 * The context is cut into splits of split_tokens tokens; each split's
 * unnormalised softmax state (running max, sum, weighted V) goes to the
 * workspace, and a reduction pass merges the splits of each (sequence, head).
 * A sequence that fits one split has its output written by the first pass.
 *
 * split_tokens = PKV_SPLIT_BALANCED instead cuts the batch's context, taken
 * as steps of a few tokens sequence after sequence, into up to 1024 nearly
 * equal ranges (one wave each per group of KV heads; each range at least 16
 * steps, and no sequence in more than 512 ranges; the waves that run on the
 * odd-numbered dies, which stream slower, take 1/16 less), chosen on the
 * device from context_lens, so that the waves of the first pass finish
 * together however the context lengths are mixed.  A range may end inside
 * one sequence and cover the start of the next.
 *
 * pkv_decode_split_tokens returns the split the library picks for a shape
 * (PKV_SPLIT_BALANCED when max_context_len > 256, else max_context_len
 * rounded up to a multiple of 64: one split per sequence); pass it, or 0 for
 * the same choice, or any positive multiple of 64, or PKV_SPLIT_BALANCED.
 * pkv_decode_workspace_bytes gives the workspace size that split needs (0
 * when no sequence can span two splits).
 */
#define PKV_SPLIT_BALANCED (-1)

int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t block_size, int32_t dtype);

int64_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t split_tokens);

/*
 *   q               [num_seqs, num_q_heads, head_dim]
 *   k_cache,v_cache [num_blocks, block_size, num_kv_heads, head_dim], read only
 *   block_tables    [num_seqs, max_blocks_per_seq] int32 physical block ids
 *   context_lens    [num_seqs] int32, 0 <= context_lens[b] <= max_context_len
 *                   (0 gives an output row of zeros)
 *   max_context_len host int, at most max_blocks_per_seq * block_size
 *   scale           softmax scale (usually 1 / sqrt(head_dim))
 *   out             [num_seqs, num_q_heads, head_dim], written; must not alias an input
 *   split_tokens    0, PKV_SPLIT_BALANCED or a positive multiple of 64
 *   workspace       device scratch of at least
 *                   pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 *                   max_context_len, split) bytes (may be NULL when that is 0);
 *                   its contents on entry do not matter.
 */
int pkv_paged_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                          float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                          int32_t split_tokens, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): pkv_paged_decode_attn with the split-K
 * states kept in a scratch array inside the library instead of a caller
 * workspace.  Same arguments, minus workspace and workspace_bytes; same
 * kernels, so the results are bit-identical to pkv_paged_decode_attn with the
 * same split_tokens.
 *
 * - The scratch is pkv_noalloc_scratch_bytes() = 64 MiB per GPU, a static
 *   device array: each GPU the library runs on holds its own copy until the
 *   process ends.  Nothing is allocated or freed by the call.
 * - A call whose split states need more than that returns PKV_ERR_WORKSPACE
 *   before anything is enqueued (raise split_tokens, or use
 *   pkv_paged_decode_attn).  The states take
 *   pkv_decode_workspace_bytes(...) bytes: with a fixed split num_seqs *
 *   num_q_heads * S * (head_dim + 2) * 4, S = ceil(max_context_len / split);
 *   token-balanced (1024 + num_seqs) * num_q_heads * (head_dim + 2) * 4 +
 *   8 * num_seqs.
 * - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (on different streams, or from several threads without
 *   ordering) race and give undefined results.  Calls ordered on one stream
 *   are safe; each call's states are written before they are read, so
 *   nothing needs clearing between calls.
 * - The device that is current on the calling thread must be the stream's
 *   (PKV_ERR_INVALID_ARG otherwise); its scratch address is looked up on the
 *   first call on that device.
 */
int pkv_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int64_t num_blocks, int32_t block_size, int32_t dtype, int32_t split_tokens,
                                  void* stream);

/* Bytes of the per-GPU scratch of pkv_paged_decode_attn_noalloc. */
int64_t pkv_noalloc_scratch_bytes(void);

/* The two passes of pkv_paged_decode_attn, enqueued separately (same
 * arguments; call split then reduce on one stream).  Together they do
 * exactly what pkv_paged_decode_attn does. */
int pkv_paged_decode_split(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                           float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                           int32_t split_tokens, void* workspace, int64_t workspace_bytes, void* stream);

int pkv_paged_decode_reduce(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                            float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                            int32_t split_tokens, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Decode with the cache write fused in: the same as pkv_kv_store of each
 * sequence's newest token followed by pkv_paged_decode_attn, in the decode
 * launch (one launch fewer per step; the pages capture the decode step in a
 * CUDA graph to cut launch costs, "Nano-vLLM Architecture and Performance",
 * section "Key Features", item "CUDA Graph Capture").
 *
 *   k, v     [num_seqs, num_kv_heads, head_dim]: the K/V rows of each
 *            sequence's newest token, the one at position context_lens[b] - 1
 *            (context_lens counts it).  It is written to that position's row
 *            of the caches: block block_tables[b][(L - 1) / block_size], row
 *            (L - 1) % block_size.  A sequence with context_lens[b] == 0 has
 *            no new token (nothing is written, its output is zeros).
 *   other arguments as pkv_paged_decode_attn; the caches are written.
 * The decode wave that owns the newest token reads it from k, v instead of
 * the cache and writes it, so results and caches are bit-identical to the
 * two separate calls.  That row must be private to the sequence (never a
 * shared prefix block).
 */
int pkv_paged_decode_store_attn(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                int32_t dtype, int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                                void* stream);

/*
 * Shared-prefix ("cascade") decode: the same result as pkv_paged_decode_attn
 * (up to rounding), for a batch in which groups of sequences begin with the
 * same cached blocks (prefix caching: blocks of a common prefix are reused
 * with reference counts, "Nano-vLLM Architecture and Performance", section
 * "Key Features", item "Paged KV Cache"; the nano-vllm README's feature list
 * names the sharing of KV blocks for common prefixes).  The shared keys
 * are read once per group instead of once per member: a group pass on the
 * matrix cores attends every member's query to the shared blocks, chunk by
 * chunk, and the split pass attends each sequence's own keys; the reduction
 * merges both kinds of softmax state with the split-K formula.
 *
 * Arguments as pkv_paged_decode_attn, plus:
 *   shared_lens    [num_seqs] int32: keys of sequence b that lie in its
 *                  group's shared blocks (a multiple of block_size, below
 *                  context_lens[b]); 0 for a sequence in no group.
 *   group_offsets  [num_groups + 1] int32, non-decreasing from 0: group gi is
 *                  group_seqs[group_offsets[gi] .. group_offsets[gi + 1]).
 *   group_seqs     sequence indices; every sequence with shared_lens > 0 is
 *                  in exactly one group; members of a group have the same
 *                  shared_lens and the same first shared_lens / block_size
 *                  block ids.
 *   max_group_size >= the largest group; max_shared_len >= every shared_lens
 *                  entry, a multiple of block_size below max_context_len.
 *   max_own_len    >= every context_lens[b] - shared_lens[b] (the keys a
 *                  sequence attends on its own); it sizes the split pass.
 *                  0 means max_context_len.
 *   split_tokens   split length of the split pass, PKV_SPLIT_BALANCED (the
 *                  own keys of the batch in token-balanced ranges, as in
 *                  pkv_paged_decode_attn), or 0 for the library's choice:
 *                  token-balanced ranges when num_seqs * max_own_len is at
 *                  least 1024 * 256 and max_own_len > 256, else splits down to
 *                  64 keys aiming at about 2048 waves.
 *   workspace      at least pkv_cascade_workspace_bytes(...) bytes (same
 *                  sizes and split_tokens as the call).
 * With num_groups == 0 or max_shared_len == 0 this is pkv_paged_decode_attn
 * (shared_lens, group_offsets and group_seqs are not read).  The group pass
 * needs dtype PKV_BF16 (PKV_ERR_UNSUPPORTED otherwise) and a scale > 0
 * (PKV_ERR_INVALID_ARG otherwise: it takes the maximum of unscaled scores and
 * masks keys past a chunk's end with -inf).  The device-side
 * preconditions above are not checked.
 */
int pkv_cascade_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                            const int32_t* shared_lens, const int32_t* group_offsets, const int32_t* group_seqs,
                            int32_t num_groups, int32_t max_group_size, int32_t max_shared_len, int32_t max_own_len,
                            float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t dtype,
                            int32_t split_tokens, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes pkv_cascade_decode_attn needs for these sizes and split_tokens
 * (0 when it writes every output directly). */
int64_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t max_own_len, int32_t split_tokens,
                                    int32_t num_groups, int32_t max_group_size, int32_t max_shared_len);

/*
 * Causal varlen prefill attention (chunked prefill and cached prefixes).
 * Sequence b has Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] new queries and
 * Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys in all, Lq <= Lk.  Query i
 * sits at position Lk - Lq + i and attends keys 0 .. Lk - Lq + i (causal: a
 * query attends keys at positions up to its own, nano-vllm README, tutorial
 * chapter "Self-Attention"; aligned to the newest token so that a chunk after
 * a cached prefix gives what full recomputation would, README section on the
 * KV cache: only the new tokens are computed).
 *
 *   q             [total_q, num_q_heads, head_dim], rows cu_seqlens_q[b] + i
 *   k, v          block_tables != NULL: the caches
 *                 [num_blocks, block_size, num_kv_heads, head_dim] (the new
 *                 tokens already stored by pkv_kv_store); block_tables == NULL:
 *                 packed [num_blocks, num_kv_heads, head_dim] rows, sequence
 *                 b's key t at row cu_seqlens_k[b] + t (num_blocks is then the
 *                 row count and block_size is ignored).
 *   cu_seqlens_q,
 *   cu_seqlens_k  [num_seqs + 1] int32, starting at 0, non-decreasing.
 *   block_tables  [num_seqs, max_blocks_per_seq] int32 or NULL.
 *   out           [total_q, num_q_heads, head_dim], written; must not alias an input.
 *   scale         softmax scale; scale <= 0 selects 1 / sqrt(head_dim).
 *   max_seqlen_q,
 *   max_seqlen_k  host bounds on Lq and Lk over the sequences.
 *
 *   workspace     NULL, or device scratch of at least
 *                 pkv_prefill_workspace_bytes(num_seqs, max_seqlen_q, num_q_heads,
 *                 num_kv_heads, head_dim, dtype) bytes, 256-byte aligned (its
 *                 contents on entry do not matter; PKV_ERR_WORKSPACE if too small).
 *
 * bf16 runs on the matrix cores (bf16 operands, fp32 accumulation, the
 * softmax weights rounded to bf16 before they multiply V); fp32 runs on the
 * vector units in fp32 and ignores the workspace.
 *
 * With a workspace (bf16), a planning kernel reads cu_seqlens on the device
 * and writes per-die work lists into it (sequences with the most keys first,
 * long query tiles cut along their keys into pieces whose partial softmax
 * states are merged in piece order, so results are deterministic), and one
 * workgroup per listed item works through them (the library can also be
 * built to walk the lists with one persistent workgroup per compute unit).
 * Without one, each query tile is a workgroup of a single launch.  Both
 * compute the same function within rounding; the split and merge change the
 * rounding order, not the result's definition.
 */
int64_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t max_seqlen_q, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

int pkv_paged_prefill_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           void* out, float scale, int32_t num_seqs, int64_t total_q, int32_t max_seqlen_q,
                           int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int64_t num_blocks, int32_t block_size, int32_t dtype, void* workspace,
                           int64_t workspace_bytes, void* stream);

/*
 * Block gather (a check of the paged addressing every kernel uses): copy the
 * Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] logical tokens of each sequence,
 * read through its block table, to rows cu_seqlens_k[b] .. of k_out / v_out
 * ([cu_seqlens_k[num_seqs], num_kv_heads, head_dim]).  Bit-exact copy
 * ("PagedAttention: Allocate blocks on-demand" diagram of the nano-vllm
 * README: a sequence's blocks need not be contiguous).
 */
int pkv_paged_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens_k, int32_t num_seqs,
                     int32_t max_seqlen_k, void* k_out, void* v_out, int32_t num_kv_heads, int32_t head_dim,
                     int64_t num_blocks, int32_t block_size, int32_t dtype, void* stream);

/*
 * Block manager (host memory only; no device work).  Hands out the physical
 * blocks of a paged KV cache and builds the block tables and slot mappings
 * the calls above consume ("Nano-vLLM Architecture and Performance", section
 * "Paged KV Cache": the cache is cut into fixed-size blocks that a block
 * manager hands out as sequences grow, and blocks holding a common prefix are
 * reused under reference counts).
 *
 * - Blocks have reference counts.  A sequence's full prompt blocks are
 *   looked up in a prefix cache keyed by a hash chained over the token ids of
 *   all blocks up to and including that one; a hit is confirmed token by
 *   token and shares the block (count + 1).  The first miss ends the lookup.
 * - A full block written by one sequence only (count 1) is registered in the
 *   cache; freed blocks (count 0) keep their registration and stay reusable
 *   until the block is handed out again for new data (free blocks are reused
 *   oldest first, and a sequence's blocks are freed last block first, so its
 *   prefix stays cached longest).  A sequence's partial last block is always
 *   its own.
 * - Slots are int32: num_blocks * block_size must be below 2^31.
 * - Each manager is internally locked; calls on one manager may come from
 *   several threads.  Errors return a negative pkv_status with text in
 *   pkv_bm_last_error() (thread-local); PKV_ERR_OUT_OF_BLOCKS leaves the
 *   manager unchanged, so a caller can preempt (pkv_bm_preempt) and retry.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager over num_blocks blocks of block_size tokens; NULL on error.
 * enable_prefix_cache = 0 turns prefix reuse off. */
pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size, int32_t enable_prefix_cache);
void pkv_bm_destroy(pkv_block_manager* bm);
const char* pkv_bm_last_error(void);

int64_t pkv_bm_num_free_blocks(pkv_block_manager* bm);
/* Reference count of a physical block (0 = free). */
int32_t pkv_bm_block_refcount(pkv_block_manager* bm, int32_t block);

/* 1 if a prompt of num_tokens token ids (host array) can be allocated now, 0 if not. */
int pkv_bm_can_allocate(pkv_block_manager* bm, const int32_t* tokens, int64_t num_tokens);

/* Allocate the blocks of a new sequence's prompt (tokens: host array of token
 * ids), reusing cached prefix blocks.  *num_cached_tokens (may be NULL)
 * receives how many leading tokens were found in the cache: their K/V are
 * already stored, so only the rest need computing and storing. */
int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int64_t num_tokens,
                    int64_t* num_cached_tokens);

/* Append one token (decode); a new block is taken when the token starts one.
 * *slot (may be NULL) receives the token's slot for pkv_kv_store. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int32_t token, int32_t* slot);

/* Release a sequence's blocks. */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);

/* Preemption when the pool runs short (nano-vLLM's scheduler evicts running
 * sequences back to its waiting queue and frees their blocks when the KV
 * cache is exhausted: "Nano-vLLM Architecture and Performance", section "Key
 * Features", item "Preemption").  Frees the blocks of the most recently
 * allocated sequence still held and forgets it; the caller keeps its tokens
 * and re-queues it.  *seq_id (may be NULL) receives its id; *num_cached_tokens
 * (may be NULL) receives how many of its leading tokens the prefix cache
 * still holds right after the free (what re-allocating it would reuse if no
 * other allocation takes those blocks first).  PKV_ERR_INVALID_ARG if no
 * sequence holds blocks. */
int pkv_bm_preempt(pkv_block_manager* bm, int64_t* seq_id, int64_t* num_cached_tokens);

/* Tokens of a sequence (its context length), or a negative status. */
int64_t pkv_bm_seq_len(pkv_block_manager* bm, int64_t seq_id);

/* Write the sequence's block table into out[0 .. capacity), padding unused
 * entries with pad; returns the number of blocks or a negative status. */
int32_t pkv_bm_block_table(pkv_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity, int32_t pad);

/* Slots of positions first_pos .. first_pos + count - 1 of a sequence. */
int pkv_bm_slot_mapping(pkv_block_manager* bm, int64_t seq_id, int64_t first_pos, int64_t count, int32_t* out);

/*
 * Precondition checks.  The attention calls check every argument they can on
 * the host, but their device-side preconditions (block ids inside the pool,
 * lengths within the stated maxima, cu_seqlens ordered with Lq <= Lk, slots
 * inside the pool and distinct, consistent shared-prefix groups) are the
 * caller's: breaking one gives undefined results, possibly a memory fault.
 * These calls test them on the device without touching the caches (they read
 * only the metadata arrays, so they are safe on any input) and leave in
 * `flags` (device int32[PKV_CHECK_NUM_FLAGS], zeroed by the call) the number
 * of violations of each kind.  Asynchronous like every call: read `flags`
 * after synchronizing the stream.  They check exactly the conditions of the
 * matching attention call with the same arguments.
 */
typedef enum {
  PKV_CHECK_LENGTH = 0,         /* a context or key count outside [0, max], or more blocks than a table row holds */
  PKV_CHECK_BLOCK_ID = 1,       /* a block id outside [0, num_blocks) among the blocks a sequence uses */
  PKV_CHECK_CU_SEQLENS = 2,     /* cu_seqlens not starting at 0 or decreasing, Lq > Lk, or above the maxima */
  PKV_CHECK_SLOT = 3,           /* a slot >= num_blocks * block_size */
  PKV_CHECK_DUPLICATE_SLOT = 4, /* a slot named by two tokens (only with a bitmap) */
  PKV_CHECK_SHARED_PREFIX = 5,  /* a member whose shared length or shared block ids differ from its group's,
                                   not whole blocks, not below its context, or above max_shared_len */
  PKV_CHECK_GROUP = 6,          /* bad group offsets or member index, or a sequence in no group (with a shared
                                   length) or in several */
  PKV_CHECK_NUM_FLAGS = 8
} pkv_check_flag;

/* Preconditions of pkv_paged_decode_attn (and of the cascade call's tables). */
int pkv_check_decode_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs, int64_t num_blocks, int32_t block_size,
                            int32_t* flags, void* stream);

/* Preconditions of pkv_paged_prefill_attn (block_tables NULL: packed k/v, no block check). */
int pkv_check_prefill_inputs(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int64_t num_blocks, int32_t block_size, int32_t* flags, void* stream);

/* Preconditions of pkv_kv_store / pkv_rope_kv_store.  bitmap: NULL (no duplicate
 * check) or device uint32[ceil(num_blocks * block_size / 32)], overwritten. */
int pkv_check_slots(const int32_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                    uint32_t* bitmap, int32_t* flags, void* stream);

/* Group preconditions of pkv_cascade_decode_attn (run pkv_check_decode_inputs
 * for its tables).  num_members = entries of group_seqs; seen: device
 * int32[num_seqs], overwritten. */
int pkv_check_cascade_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             const int32_t* shared_lens, const int32_t* group_offsets, const int32_t* group_seqs,
                             int32_t num_groups, int32_t num_members, int32_t num_seqs, int32_t max_group_size,
                             int32_t max_shared_len, int32_t block_size, int32_t* seen, int32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
