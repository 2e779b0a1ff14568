// kv_store and the block gather: 16-byte copies of token rows between packed
// [tokens, Hkv, D] buffers and the paged [num_blocks, block_size, Hkv, D]
// caches.  Both move stored bits only.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

// One thread per 16-byte chunk of a token's K row and the same chunk of its V
// row.  A token row is Hkv * D * elt bytes, contiguous in the packed input and
// at slot * row_bytes in the cache (the cache is [blocks * block_size] rows),
// so the slot is the row index: no block arithmetic is needed.
// Threads: x = chunk within the row, y = token; grid x = token groups, grid y = chunk groups.
__global__ __launch_bounds__(256) void kv_store_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                       uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int64_t num_tokens, int32_t chunks_per_row) {
  const int64_t token = (int64_t)blockIdx.x * blockDim.y + threadIdx.y;
  const int32_t chunk = blockIdx.y * blockDim.x + threadIdx.x;
  if (token >= num_tokens || chunk >= chunks_per_row) return;
  const int32_t slot = slot_mapping[token];
  if (slot < 0) return;
  const int64_t src = token * chunks_per_row + chunk;
  const int64_t dst = (int64_t)slot * chunks_per_row + chunk;
  const uint4 kk = k[src];
  const uint4 vv = v[src];
  k_cache[dst] = kk;
  v_cache[dst] = vv;
}

// Gather: grid (token tiles, sequences).  Token t of sequence b is read from
// block block_tables[b][t / block_size], row t % block_size, and written to
// packed row cu_seqlens_k[b] + t.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ k_cache,
                                                     const uint4* __restrict__ v_cache,
                                                     const int32_t* __restrict__ block_tables,
                                                     int32_t max_blocks_per_seq,
                                                     const int32_t* __restrict__ cu_seqlens_k, uint4* __restrict__ k_out,
                                                     uint4* __restrict__ v_out, int32_t chunks_per_row,
                                                     int32_t log2_block_size, int32_t tokens_per_wg) {
  const int b = blockIdx.y;
  const int32_t k0 = cu_seqlens_k[b];
  const int32_t len = cu_seqlens_k[b + 1] - k0;
  const int32_t t_begin = blockIdx.x * tokens_per_wg;
  const int32_t t_end = min(len, t_begin + tokens_per_wg);
  const int32_t bs_mask = (1 << log2_block_size) - 1;
  const int32_t* table = block_tables + (int64_t)b * max_blocks_per_seq;
  for (int32_t i = threadIdx.x; i < (t_end - t_begin) * chunks_per_row; i += blockDim.x) {
    const int32_t t = t_begin + i / chunks_per_row;
    const int32_t c = i % chunks_per_row;
    const int64_t block = table[t >> log2_block_size];
    const int64_t row = (block << log2_block_size) + (t & bs_mask);
    const int64_t src = row * chunks_per_row + c;
    const int64_t dst = (int64_t)(k0 + t) * chunks_per_row + c;
    k_out[dst] = k_cache[src];
    v_out[dst] = v_cache[src];
  }
}

hipError_t launch_kv_store(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                           int64_t num_tokens, int32_t row_bytes, hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  dim3 block(64, 4);
  if (chunks < 64) block = dim3(chunks, 256 / chunks);
  dim3 grid((unsigned)((num_tokens + block.y - 1) / block.y), (chunks + block.x - 1) / block.x);
  hipLaunchKernelGGL(kv_store_kernel, grid, block, 0, stream, (const uint4*)k, (const uint4*)v, (uint4*)k_cache,
                     (uint4*)v_cache, slot_mapping, num_tokens, chunks);
  return hipGetLastError();
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* cu_seqlens_k, int32_t num_seqs,
                         int32_t max_seqlen_k, void* k_out, void* v_out, int32_t row_bytes, int32_t log2_block_size,
                         hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  const int32_t tokens_per_wg = 16;
  dim3 grid((max_seqlen_k + tokens_per_wg - 1) / tokens_per_wg, num_seqs);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, stream, (const uint4*)k_cache, (const uint4*)v_cache,
                     block_tables, max_blocks_per_seq, cu_seqlens_k, (uint4*)k_out, (uint4*)v_out, chunks,
                     log2_block_size, tokens_per_wg);
  return hipGetLastError();
}

}  // namespace pkv
