// Work lists of the persistent prefill, built on the device from cu_seqlens
// (one workgroup; the host knows only the maxima of the lengths).
//
// Items.  A query tile (qp positions of one sequence x the query heads of one
// KV head, a "pair" (sequence, head group)) needs the key tiles up to its last
// position.  A query tile with more than `cap` key tiles is cut along its
// keys into pieces of cap tiles and a last piece that holds the diagonal;
// interior cuts lie at or below the tile's first position, so every position
// sees at least one key of every piece.  cap is the smallest that leaves a
// die with about kPlanItemsPerCu maximal pieces per workgroup (at least
// kPlanMinCap tiles).
//
// Order.  Sequences are ranked by their key tiles, most first; pair (rank r,
// head group h) gets index r * nhg + h and runs on die index % 8, so the
// largest pairs are dealt round-robin over the dies.  A die's list holds its
// pairs in index order, each pair's query tiles from the last (most keys) to
// the first, a tile's pieces in key order.  Items of one pair are adjacent,
// so the workgroups of a die read the same K/V tiles through its L2 at about
// the same time; the lists end with the smallest tiles of the smallest
// pairs, which evens out the finishing times of the workgroups.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kKT = 128;  // keys per tile of the prefill kernel
constexpr int kNV = kPlanXcds + 2;  // scanned per pair: items on each die, split tiles, state slots

// key tiles query tile qt needs (up to its last position)
__device__ __forceinline__ int tiles_of(int shift, int lq, int qp, int qt) {
  const int max_pos = shift + min(qt * qp + qp, lq) - 1;
  return max(max_pos, 0) / kKT + 1;
}

// pieces of a query tile of n_kt key tiles whose first position is min_pos
__device__ __forceinline__ int pieces_of(int n_kt, int min_pos, int cap) {
  return 1 + min(max(min_pos, 0) / kKT / cap, (n_kt - 1) / cap);
}

// Everything but the item records stays in LDS (the sequences' lengths and
// per-sequence counts, kPlanMaxSeqs at most), so the phases cost barriers,
// not memory round trips.
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillPlanArgs p) {
  __shared__ int32_t s_scan[kNV][kPlanThreads];
  __shared__ int32_t s_cq[kPlanMaxSeqs + 1], s_ck[kPlanMaxSeqs + 1];
  __shared__ int32_t s_work[kPlanMaxSeqs], s_items[kPlanMaxSeqs], s_splits[kPlanMaxSeqs], s_slots[kPlanMaxSeqs];
  __shared__ int32_t s_rank[kPlanMaxSeqs];  // sequence of each rank
  __shared__ unsigned long long s_tiles[kPlanXcds];
  __shared__ int32_t s_cap, s_overflow;
  const int tid = threadIdx.x;
  const int B = p.num_seqs, qp = p.qp, nhg = p.nhg;
  for (int i = tid; i <= B; i += kPlanThreads) {
    s_cq[i] = p.cu_seqlens_q[i];
    s_ck[i] = p.cu_seqlens_k[i];
  }
  if (tid < kPlanXcds) s_tiles[tid] = 0;
  if (tid == 0) s_overflow = 0;
  __syncthreads();
  auto shape = [&](int b, int& lq, int& lk) {
    lq = max(s_cq[b + 1] - s_cq[b], 0);
    lk = max(s_ck[b + 1] - s_ck[b], 0);
  };

  // 1. key tiles of each sequence, summed over its query tiles
  for (int b = tid; b < B; b += kPlanThreads) {
    int lq, lk;
    shape(b, lq, lk);
    const int nqt = (lq + qp - 1) / qp;
    long long w = 0;
    for (int qt = 0; qt < nqt; ++qt) w += tiles_of(lk - lq, lq, qp, qt);
    s_work[b] = (int32_t)min(w, (long long)INT_MAX);
  }
  __syncthreads();

  // 2. rank: most key tiles first, ties by index
  for (int b = tid; b < B; b += kPlanThreads) {
    const int w = s_work[b];
    int r = 0;
    for (int c = 0; c < B; ++c) r += (s_work[c] > w) || (s_work[c] == w && c < b);
    s_rank[r] = b;
  }
  __syncthreads();

  // 3. key tiles per die (pair (rank r, head group h) has index r * nhg + h and
  // runs on die index % 8), and the piece cap
  for (int r = tid; r < B; r += kPlanThreads) {
    const unsigned long long w = (unsigned long long)s_work[s_rank[r]];
    for (int h = 0; h < nhg; ++h) atomicAdd(&s_tiles[((int64_t)r * nhg + h) % kPlanXcds], w);
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long mx = 0;
    for (int x = 0; x < kPlanXcds; ++x) mx = max(mx, s_tiles[x]);
    const unsigned long long per = (unsigned long long)kPlanItemsPerCu * kPlanCusPerXcd;
    s_cap = (int)min(max((mx + per - 1) / per, (unsigned long long)kPlanMinCap), (unsigned long long)INT_MAX);
  }
  __syncthreads();
  const int cap = s_cap;

  // 4. items, split query tiles and state slots of each sequence (the same for each head group)
  for (int b = tid; b < B; b += kPlanThreads) {
    int lq, lk;
    shape(b, lq, lk);
    const int nqt = (lq + qp - 1) / qp;
    int items = 0, splits = 0, slots = 0;
    for (int qt = 0; qt < nqt; ++qt) {
      const int nc = pieces_of(tiles_of(lk - lq, lq, qp, qt), lk - lq + qt * qp, cap);
      items += nc;
      if (nc > 1) {
        ++splits;
        slots += nc;
      }
    }
    s_items[b] = items;
    s_splits[b] = splits;
    s_slots[b] = slots;
  }
  __syncthreads();

  // 5. exclusive scans over the pairs in index order
  const int64_t P = (int64_t)B * nhg;
  const int64_t per_t = (P + kPlanThreads - 1) / kPlanThreads;
  const int64_t p0 = min(P, (int64_t)tid * per_t), p1 = min(P, p0 + per_t);
  int32_t acc[kNV];
#pragma unroll
  for (int v = 0; v < kNV; ++v) acc[v] = 0;
  for (int64_t pp = p0; pp < p1; ++pp) {
    const int b = s_rank[pp / nhg];
    acc[pp % kPlanXcds] += s_items[b];
    acc[kPlanXcds] += s_splits[b];
    acc[kPlanXcds + 1] += s_slots[b];
  }
#pragma unroll
  for (int v = 0; v < kNV; ++v) s_scan[v][tid] = acc[v];
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {
    int32_t t[kNV];
#pragma unroll
    for (int v = 0; v < kNV; ++v) t[v] = tid >= d ? s_scan[v][tid - d] : 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < kNV; ++v) s_scan[v][tid] += t[v];
    __syncthreads();
  }
  int32_t off[kNV];
#pragma unroll
  for (int v = 0; v < kNV; ++v) off[v] = s_scan[v][tid] - acc[v];

  // 6. the item records
  bool overflow = false;
  for (int64_t pp = p0; pp < p1; ++pp) {
    const int h = (int)(pp % nhg);
    const int x = (int)(pp % kPlanXcds);
    const int b = s_rank[pp / nhg];
    int lq, lk;
    shape(b, lq, lk);
    const int nqt = (lq + qp - 1) / qp;
    for (int qt = nqt - 1; qt >= 0; --qt) {
      const int n_kt = tiles_of(lk - lq, lq, qp, qt);
      const int nc = pieces_of(n_kt, lk - lq + qt * qp, cap);
      int split = -1, slot = 0;
      bool ok = true;
      if (nc > 1) {
        split = off[kPlanXcds]++;
        slot = off[kPlanXcds + 1];
        off[kPlanXcds + 1] += nc;
        ok = split < p.split_cap && slot + nc <= p.slot_cap;
      }
      for (int c = 0; c < nc; ++c) {
        const int idx = off[x]++;
        if (!ok || idx >= p.items_cap) {
          overflow = true;
          continue;
        }
        int4* rec = reinterpret_cast<int4*>(p.items + ((int64_t)x * p.items_cap + idx) * kItemInts);
        rec[0] = make_int4(b, h, qt, c * cap);
        rec[1] = make_int4(c + 1 < nc ? (c + 1) * cap : n_kt, c | (nc << 16), split, slot);
      }
    }
  }
  if (overflow) atomicOr(&s_overflow, 1);
  __syncthreads();

  // 7. header: queue heads start past the items every workgroup takes by its
  // index, item counts, and the arrival counters (one per split tile and wave) zeroed
  const int splits = min(s_scan[kPlanXcds][kPlanThreads - 1], p.split_cap) * kPlanWaves;
  if (tid < kPlanXcds) {
    p.hdr[tid] = kPlanStaticItems * kPlanCusPerXcd;
    p.hdr[kPlanXcds + tid] = min(s_scan[tid][kPlanThreads - 1], p.items_cap);
  }
  if (tid == 0) {
    p.hdr[kHdrCap] = cap;
    p.hdr[kHdrOverflow] = s_overflow;
    p.hdr[kHdrSplits] = s_scan[kPlanXcds][kPlanThreads - 1];
    p.hdr[kHdrSlots] = s_scan[kPlanXcds + 1][kPlanThreads - 1];
  }
  for (int i = tid; i < splits; i += kPlanThreads) p.arrive[i] = 0;
}

}  // namespace

hipError_t launch_prefill_plan(const PrefillPlanArgs& p, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
