// Validation kernels for the device-side preconditions of the attention calls.
// They read only metadata (block tables, lengths, cu_seqlens, slots, groups),
// never the caches, so they are safe to run on any input; each violation adds
// one to its counter in the caller's flags array (zeroed first by the same
// call, with a fill kernel so that the call can sit in a captured graph).
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

__global__ __launch_bounds__(64) void zero_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 64) p[i] = 0;
}

__device__ __forceinline__ void flag(int32_t* flags, int code) { atomicAdd(flags + code, 1); }

// One workgroup per sequence: its key count (decode: context_lens; prefill:
// cu_seqlens_k difference) within bounds, and the block ids that hold those
// keys inside the pool.  Prefill also checks cu_seqlens (non-decreasing, Lq <= Lk,
// the stated maxima).
__global__ __launch_bounds__(256) void check_tables_kernel(CheckArgs a) {
  const int b = blockIdx.x;
  int L;
  if (a.context_lens) {
    L = a.context_lens[b];
    if (L < 0 || L > a.max_len_k) {
      if (threadIdx.x == 0) flag(a.flags, kCheckLength);
      return;
    }
  } else {
    const int q0 = a.cu_seqlens_q[b], q1 = a.cu_seqlens_q[b + 1];
    const int k0 = a.cu_seqlens_k[b], k1 = a.cu_seqlens_k[b + 1];
    const int lq = q1 - q0;
    L = k1 - k0;
    const bool bad = q0 < 0 || k0 < 0 || lq < 0 || L < 0 || lq > L || lq > a.max_len_q || L > a.max_len_k ||
                     (b == 0 && (q0 != 0 || k0 != 0));
    if (bad) {
      if (threadIdx.x == 0) flag(a.flags, kCheckCuSeqlens);
      return;
    }
  }
  if (!a.block_tables) return;
  const int64_t nblk = ((int64_t)L + a.block_size - 1) / a.block_size;
  if (nblk > a.max_blocks_per_seq) {
    if (threadIdx.x == 0) flag(a.flags, kCheckLength);
    return;
  }
  const int32_t* row = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  int bad = 0;
  for (int i = threadIdx.x; i < (int)nblk; i += blockDim.x) bad += (row[i] < 0 || row[i] >= a.num_blocks);
  if (bad) atomicAdd(a.flags + kCheckBlockId, bad);
}

// One thread per token: slot inside the pool; with a bitmap, a slot named twice.
__global__ __launch_bounds__(256) void check_slots_kernel(CheckArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.num_tokens) return;
  const int32_t s = a.slot_mapping[i];
  if (s < 0) return;  // skipped token
  if ((int64_t)s >= a.num_blocks * a.block_size) {
    flag(a.flags, kCheckSlot);
    return;
  }
  if (a.bitmap) {
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(a.bitmap + (s >> 5), bit) & bit) flag(a.flags, kCheckDuplicateSlot);
  }
}

// One workgroup per group: members' shared lengths equal, whole blocks, below
// their contexts and within max_shared_len; their first shared blocks equal the
// first member's; each member counted once in `seen` (sequences in several
// groups are then caught by the membership pass below).
__global__ __launch_bounds__(256) void check_groups_kernel(CheckArgs a) {
  const int gi = blockIdx.x;
  const int m0 = a.group_offsets[gi], m1 = a.group_offsets[gi + 1];
  if (m0 < 0 || m1 < m0 || m1 > a.num_members || m1 - m0 > a.max_group_size || (gi == 0 && m0 != 0)) {
    if (threadIdx.x == 0) flag(a.flags, kCheckGroup);
    return;
  }
  if (m1 == m0) return;
  const int first = a.group_seqs[m0];
  if (first < 0 || first >= a.num_seqs) {
    if (threadIdx.x == 0) flag(a.flags, kCheckGroup);
    return;
  }
  const int sh = a.shared_lens[first];
  const int nblk = sh / a.block_size;
  const int32_t* row0 = a.block_tables + (int64_t)first * a.max_blocks_per_seq;
  for (int m = m0 + (int)threadIdx.x / 64; m < m1; m += blockDim.x / 64) {
    const int lane = threadIdx.x % 64;
    const int b = a.group_seqs[m];
    if (b < 0 || b >= a.num_seqs) {
      if (lane == 0) flag(a.flags, kCheckGroup);
      continue;
    }
    if (lane == 0) {
      atomicAdd(a.seen + b, 1);
      const int L = a.context_lens[b];
      if (a.shared_lens[b] != sh || sh <= 0 || sh % a.block_size || sh >= L || sh > a.max_shared_len ||
          nblk > a.max_blocks_per_seq)
        flag(a.flags, kCheckSharedPrefix);
    }
    if (nblk > a.max_blocks_per_seq) continue;
    const int32_t* row = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
    int bad = 0;
    for (int i = lane; i < nblk; i += 64) bad += row[i] != row0[i];
    if (bad) atomicAdd(a.flags + kCheckSharedPrefix, bad);
  }
}

// Every sequence with a shared prefix is in exactly one group, every other in none.
__global__ __launch_bounds__(256) void check_membership_kernel(CheckArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.num_seqs) return;
  const int want = a.shared_lens[b] > 0 ? 1 : 0;
  if (a.seen[b] != want) flag(a.flags, kCheckGroup);
}

}  // namespace

hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 63) / 64;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_check_tables(const CheckArgs& a, hipStream_t stream) {
  if (a.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_tables_kernel, dim3((unsigned)a.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_check_slots(const CheckArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((a.num_tokens + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_check_groups(const CheckArgs& a, hipStream_t stream) {
  if (a.num_groups > 0) {
    hipLaunchKernelGGL(check_groups_kernel, dim3((unsigned)a.num_groups), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_membership_kernel, dim3((unsigned)((a.num_seqs + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
