// Row attention on the vector units: one wave = one query row of every head
// of HPW KV heads, streaming that row's keys through the block table.
//
//  * Decode: a row is sequence b's new token.  Its context is cut into splits
//    of split_tokens keys, one wave per (sequence, KV-head group, split), or
//    (token-balanced) the batch's contexts are cut into nearly equal ranges
//    that may cross sequences, one wave per (range, KV-head group).  A part
//    of a context writes an unnormalised softmax state that decode_reduce
//    merges.
//  * Prefill rows (fp32 path): query i of sequence b attends keys 0..p with
//    p = Lk - Lq + i, in one split.
//
// Lane layout: the 64 lanes are HPW groups of TL = 64 / HPW lanes, one group
// per KV head.  Lane c of a group owns DPL = D / TL elements of the head
// dimension, as NCH chunks of CH bytes: chunk jj covers elements
// [(jj * TL + c) * EPC, +EPC).  A load instruction then reads, for every head
// of the group, TL * CH contiguous bytes of the token's row.  Each K/V byte is
// loaded once and used for all G query heads that share the KV head (their
// queries sit in the same lanes).
//
// Per step of U tokens: partial dot products per lane (bf16: v_dot2 on packed
// pairs), an all-reduce over the TL lanes of the group with DPP, the online
// softmax update (max in log2 units; the running reference max is only raised
// when a score exceeds it by more than kTau, which keeps the weights <= 2^kTau
// and skips most rescales), then weights times V accumulated in fp32.  For
// bf16 the weights are rounded to bf16 and two tokens go through one v_dot2
// per element; the weight sum is taken over the same rounded weights.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

template <int CH>
struct Chunk;
template <>
struct Chunk<16> {
  typedef uint4 type;
};
template <>
struct Chunk<8> {
  typedef uint2 type;
};
template <>
struct Chunk<4> {
  typedef uint32_t type;
};

template <int CH>
__device__ __forceinline__ void load_words(uint32_t* w, const char* p) {
  typedef typename Chunk<CH>::type T;
  T x = *reinterpret_cast<const T*>(p);
  if constexpr (CH == 16) {
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (CH == 8) {
    w[0] = x.x; w[1] = x.y;
  } else {
    w[0] = x;
  }
}

// K/V stream loads: each byte is read once per launch, so they are marked
// non-temporal (they then do not evict cache lines that other data reuses;
// measured 2-14 % faster than ordinary loads on every decode shape).
#ifndef PKV_ROW_NT
#define PKV_ROW_NT 1
#endif
template <int CH>
__device__ __forceinline__ void load_stream(uint32_t* w, const char* p) {
  if constexpr (PKV_ROW_NT != 0) {
    typedef uint32_t vec_t __attribute__((ext_vector_type(CH / 4)));
    const vec_t x = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(p));
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) w[i] = x[i];
  } else {
    load_words<CH>(w, p);
  }
}

template <int CH>
__device__ __forceinline__ void store_words(char* p, const uint32_t* w) {
  typedef typename Chunk<CH>::type T;
  T x;
  if constexpr (CH == 16) {
    x.x = w[0]; x.y = w[1]; x.z = w[2]; x.w = w[3];
  } else if constexpr (CH == 8) {
    x.x = w[0]; x.y = w[1];
  } else {
    x = w[0];
  }
  *reinterpret_cast<T*>(p) = x;
}

// Wave-wide sum (64 lanes).
__device__ __forceinline__ long long wave_sum_i64(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Token-balanced decode (see RowAttnArgs): sequence b is n_b = max(1,
// ceil((L_b - kv_start_b) / U)) steps of U tokens over its own keys (an empty
// context counts one step, which writes its row of zeros); the batch's N
// steps, sequence after sequence, are cut into W <= N ranges (none empty),
// wave w taking [start(w), start(w + 1)).  A range may cross sequences: each
// (wave, sequence) pair it touches is a segment, whose state goes to slot
// w + b.  Along the step order w + b grows by at least one per segment, so
// the segments of one sequence sit in consecutive slots, all below W + B.
//
// The ranges are not quite equal.  Workgroup w runs on die w % 8 (the
// dispatcher deals workgroups to the 8 dies in turn), and per-wave timestamps
// show the waves of the odd-numbered dies streaming 5-11 % slower than those
// of the even-numbered ones on every box measured; so the waves of odd w get
// 1/16 less than the mean range and those of even w 1/16 more:
// start(w) = floor(N (64 w + kOddDieShare (w mod 2)) / (64 W)).  (Where the
// dies run alike, this costs at most 1/16 of the launch.)
constexpr long long kOddDieShare = 4;  // in 64ths of a mean range
__device__ __forceinline__ long long steps_of(int L, int U) { return max(1, (max(L, 0) + U - 1) / U); }
// first step of wave w's range (N for w = W)
__device__ __forceinline__ long long range_start(int w, long long N, int W) {
  if (w >= W) return N;
  return N * (64LL * w + kOddDieShare * (w & 1)) / (64LL * W);
}
// the wave whose range holds step x, 0 <= x < N: the equal split's wave, moved
// by at most one (the ranges differ from the equal split's by under one range)
__device__ __forceinline__ int wave_of_step(long long x, long long N, int W) {
  int w = (int)(((x + 1) * (long long)W - 1) / N);
  while (w > 0 && range_start(w, N, W) > x) --w;
  while (w + 1 < W && range_start(w + 1, N, W) <= x) ++w;
  return w;
}
__device__ __forceinline__ long long readlane_i64(long long x, int src) {
  const int lo = __builtin_amdgcn_readlane((int)(unsigned)(x & 0xffffffffLL), src);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), src);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ long long wave_inclusive_scan_i64(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}
// Total steps N of the batch, and the sequence b holding step s (< N) with
// its first step base, which every wave derives from context_lens.  The
// lengths are read kScanBatch * 64 at a time (one memory round trip for that
// many sequences); the first batch's stay in registers for the search.
constexpr int kScanBatch = 4;
struct StepScan {
  int L[kScanBatch];        // context lengths of sequences lane + 64 k
  int st[kScanBatch];       // their first own key (kv_start, else 0)
  long long n[kScanBatch];  // their steps (0 past the end)
};
__device__ __forceinline__ void scan_load(const RowAttnArgs& a, int U, int i0, int lane, StepScan& sc) {
#pragma unroll
  for (int k = 0; k < kScanBatch; ++k) {
    const int i = i0 + 64 * k + lane;
    sc.L[k] = i < a.num_seqs ? max(a.context_lens[i], 0) : 0;
    sc.st[k] = (i < a.num_seqs && a.kv_start) ? a.kv_start[i] : 0;
  }
#pragma unroll
  for (int k = 0; k < kScanBatch; ++k)
    sc.n[k] = i0 + 64 * k + lane < a.num_seqs ? steps_of(sc.L[k] - sc.st[k], U) : 0;
}
// N, and the most steps of any one sequence in nmax.
__device__ __forceinline__ long long total_steps(const RowAttnArgs& a, int U, int lane, StepScan& first,
                                                 long long& nmax) {
  long long n = 0, mx = 0;
  scan_load(a, U, 0, lane, first);
#pragma unroll
  for (int k = 0; k < kScanBatch; ++k) {
    n += first.n[k];
    mx = max(mx, first.n[k]);
  }
  for (int i0 = 64 * kScanBatch; i0 < a.num_seqs; i0 += 64 * kScanBatch) {
    StepScan sc;
    scan_load(a, U, i0, lane, sc);
#pragma unroll
    for (int k = 0; k < kScanBatch; ++k) {
      n += sc.n[k];
      mx = max(mx, sc.n[k]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (long long)__shfl_xor(mx, o));
  nmax = mx;
  return wave_sum_i64(n);
}
// Waves of a token-balanced launch: at most W, at least kMinSteps steps each
// (shorter ranges cost more in per-wave start-up and states than they save),
// and no sequence cut into more than kMaxParts parts (its merge reads at most
// 64 states per wave of the reduction).  Never more than N, so no range is
// empty.
constexpr int kMinSteps = 16;
constexpr int kMaxParts = 512;
__device__ __forceinline__ int balanced_waves(int W, long long N, long long nmax) {
  long long w = min((long long)W, max(1LL, N / kMinSteps));
  w = min(w, max(1LL, kMaxParts * N / max(nmax, 1LL)));
  return (int)min(w, N);
}
__device__ __forceinline__ bool sequence_of_step(const RowAttnArgs& a, int U, long long s, int lane,
                                                 const StepScan& first, int& b, long long& base, int& L,
                                                 int& start) {
  long long run = 0;
  StepScan sc = first;
  for (int i0 = 0; i0 < a.num_seqs; i0 += 64 * kScanBatch) {
    if (i0 > 0) scan_load(a, U, i0, lane, sc);
#pragma unroll
    for (int k = 0; k < kScanBatch; ++k) {
      const long long n = sc.n[k];
      const long long incl = wave_inclusive_scan_i64(n, lane);
      const long long off = run + incl - n;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(n > 0 && off <= s && s < off + n);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        b = i0 + 64 * k + src;
        base = readlane_i64(off, src);
        L = __builtin_amdgcn_readlane(sc.L[k], src);
        start = __builtin_amdgcn_readlane(sc.st[k], src);
        return true;
      }
      run += readlane_i64(incl, 63);
    }
  }
  return false;
}

// STORE: decode with the newest token's cache write fused in (k_new / v_new).
template <bool BF16, int D, int HPW, int G, int U, int R, bool PREFILL, bool STORE>
__global__ __launch_bounds__(64) void row_attn_kernel(RowAttnArgs a) {
  constexpr int ELT = BF16 ? 2 : 4;
  constexpr int TL = 64 / HPW;
  constexpr int DPL = D / TL;
  constexpr int LANE_BYTES = DPL * ELT;
  static_assert(LANE_BYTES >= 4, "a lane must own at least one 32-bit word");
  constexpr int CH = LANE_BYTES >= 16 ? 16 : LANE_BYTES;
  constexpr int NCH = LANE_BYTES / CH;
  constexpr int WPC = CH / 4;     // words per chunk
  constexpr int NW = NCH * WPC;   // words per lane per row
  constexpr int EPW = 4 / ELT;    // elements per word
  constexpr int EPC = CH / ELT;   // elements per chunk

  const int lane = threadIdx.x;
  const int hl = lane / TL;
  const int c = lane % TL;
  const int n_hg = a.num_kv_heads / HPW;
  int item = blockIdx.x;
  const int hg = item % n_hg;
  item /= n_hg;
  const int g = hg * HPW + hl;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int64_t row_bytes = (int64_t)Hkv * D * ELT;
  const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
  static_assert(!BF16 || U % 2 == 0, "bf16 steps pair tokens");

  // Zeros for the G query heads of this lane group (a decode row with an empty context).
  auto write_zeros = [&](int64_t q_row) {
    for (int gq = 0; gq < G; ++gq) {
      char* op = (char*)a.out + ((q_row * Hq + g * G + gq) * D) * ELT + c * CH;
      uint32_t z[WPC] = {};
      for (int jj = 0; jj < NCH; ++jj) store_words<CH>(op + jj * TL * CH, z);
    }
  };

  // One segment: keys [t0, t1) of query row q_row (sequence b; prefill rows
  // read packed rows from k0).  nstates == 1: the normalised output is
  // written; else the unnormalised state goes to slots sbase + (query head) *
  // sstride.  L_store: the context length, for the fused store of the newest
  // token (decode with STORE only).
  auto segment = [&](int b, int64_t q_row, int t0, int t1, int k0, int L_store, int nstates, int64_t sbase,
                     int sstride) {
    int t_new = -1;  // fused store: position of the newest token if this segment holds it
    int t_fin = -1;  // fused store: first token of the step that holds it
    if constexpr (STORE && !PREFILL) {
      if (t1 == L_store) {
        // the step holding the newest token is taken out of the streaming loop
        // and done after it, with that token read from k_new / v_new
        t_new = L_store - 1;
        t_fin = t0 + (t_new - t0) / U * U;
        t1 = t_fin;
      }
    }

    // Queries of the G heads sharing KV head g, in this lane's element order.
    // Scores are scaled by c >= 0 (a negative scale is applied by negating q,
    // which is exact, and using |c|).
    uint32_t qw[G][NW];
    for (int gq = 0; gq < G; ++gq) {
      const char* qp = (const char*)a.q + ((q_row * Hq + g * G + gq) * D) * ELT + c * CH;
      for (int jj = 0; jj < NCH; ++jj) load_words<CH>(&qw[gq][jj * WPC], qp + jj * TL * CH);
    }
    float cs = a.scale_log2;
    if (cs < 0.f) {
      const uint32_t sign = BF16 ? 0x80008000u : 0x80000000u;
      for (int gq = 0; gq < G; ++gq)
        for (int w = 0; w < NW; ++w) qw[gq][w] ^= sign;
      cs = -cs;
    }

    float m[G], l[G], o[G][DPL];
    for (int gq = 0; gq < G; ++gq) {
      m[gq] = kNegInf;
      l[gq] = 0.f;
      for (int e = 0; e < DPL; ++e) o[gq][e] = 0.f;
    }

    const int32_t* table = a.block_tables ? a.block_tables + (int64_t)b * a.max_blocks_per_seq : nullptr;
    const int bs_mask = (1 << a.log2_block_size) - 1;
    const char* kbase = (const char*)a.k;
    const char* vbase = (const char*)a.v;
    const int lane_off = g * D * ELT + c * CH;

    // Row index of the first token of a step (U tokens never straddle a block:
    // steps start at multiples of U and U divides the block size).  Block ids
    // come from a 64-entry window of the table held one per lane and read with
    // readlane, so a lookup costs no memory round trip; the window moves when a
    // step leaves it.
    int win0 = -(1 << 30);  // first block index of the window
    int win = 0;          // this lane's entry: table[win0 + lane]
    auto step_row = [&](int t) -> int64_t {
      if (table) {
        const int bi = t >> a.log2_block_size;
        if (bi - win0 >= 64 || bi < win0) {
          win0 = bi;
          const int e = bi + lane;
          win = e < a.max_blocks_per_seq ? table[e] : 0;
        }
        const int64_t blk = __builtin_amdgcn_readlane(win, bi - win0);
        return (blk << a.log2_block_size) + (t & bs_mask);
      }
      return (int64_t)k0 + t;
    };

    struct Buf {
      uint32_t k[U][NW];
      uint32_t v[U][NW];
    };
    auto load = [&](Buf& buf, int t) {
      const int64_t r0 = step_row(t);
      const int last = t1 - 1 - t;  // tokens past the end re-read the last valid row
      for (int u = 0; u < U; ++u) {
        const int64_t r = r0 + min(u, last);
        const char* kp = kbase + r * row_bytes + lane_off;
        const char* vp = vbase + r * row_bytes + lane_off;
        for (int jj = 0; jj < NCH; ++jj) {
          load_stream<CH>(&buf.k[u][jj * WPC], kp + jj * TL * CH);
          load_stream<CH>(&buf.v[u][jj * WPC], vp + jj * TL * CH);
        }
      }
    };
    auto compute = [&](const Buf& buf, int t) {
      float s[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int gq = 0; gq < G; ++gq) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            if constexpr (BF16) {
              acc = dot2_bf16(qw[gq][w], buf.k[u][w], acc);
            } else {
              acc = fmaf(__uint_as_float(qw[gq][w]), __uint_as_float(buf.k[u][w]), acc);
            }
          }
          s[u][gq] = group_sum<TL>(acc) * cs;
        }
      }
      // tokens past the end (last step only): they take token 0's score for the
      // max and get weight 0 below
      const int nvalid = t1 - t;
      if (nvalid < U) {
#pragma unroll
        for (int u = 1; u < U; ++u)
          if (u >= nvalid)
#pragma unroll
            for (int gq = 0; gq < G; ++gq) s[u][gq] = s[0][gq];
      }
      bool raise = false;
      float mx[G];
#pragma unroll
      for (int gq = 0; gq < G; ++gq) {
        mx[gq] = s[0][gq];
#pragma unroll
        for (int u = 1; u < U; ++u) mx[gq] = fmaxf(mx[gq], s[u][gq]);
        raise |= mx[gq] > m[gq] + kTau;
      }
      if (wave_any(raise)) {
#pragma unroll
        for (int gq = 0; gq < G; ++gq) {
          const float mn = fmaxf(m[gq], mx[gq]);
          const float alpha = exp2_hw(m[gq] - mn);
          m[gq] = mn;
          l[gq] *= alpha;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[gq][e] *= alpha;
        }
      }
      float p[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int gq = 0; gq < G; ++gq) p[u][gq] = exp2_hw(s[u][gq] - m[gq]);  // the max token gets exactly 1
      if (nvalid < U) {
#pragma unroll
        for (int u = 1; u < U; ++u)
          if (u >= nvalid)
#pragma unroll
            for (int gq = 0; gq < G; ++gq) p[u][gq] = 0.f;
      }
      if constexpr (BF16) {
        // weights of two tokens as one bf16 pair; V of the two tokens interleaved
        // per element, so each v_dot2 adds both tokens' terms of one element.
#pragma unroll
        for (int u = 0; u < U; u += 2) {
          uint32_t pp[G];
#pragma unroll
          for (int gq = 0; gq < G; ++gq) {
            pp[gq] = pack_bf16x2(p[u][gq], p[u + 1][gq]);
            l[gq] = dot2_bf16(pp[gq], kOnes, l[gq]);
          }
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            // v_perm_b32: selector bytes 0-3 pick from the second operand, 4-7 from the first
            const uint32_t a0 = buf.v[u][w], a1 = buf.v[u + 1][w];
            const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // (a0.lo, a1.lo)
            const uint32_t hi = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // (a0.hi, a1.hi)
#pragma unroll
            for (int gq = 0; gq < G; ++gq) {
              o[gq][2 * w] = dot2_bf16(pp[gq], lo, o[gq][2 * w]);
              o[gq][2 * w + 1] = dot2_bf16(pp[gq], hi, o[gq][2 * w + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int gq = 0; gq < G; ++gq) l[gq] += p[u][gq];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const float v0 = __uint_as_float(buf.v[u][w]);
#pragma unroll
            for (int gq = 0; gq < G; ++gq) o[gq][w] = fmaf(p[u][gq], v0, o[gq][w]);
          }
        }
      }
    };

    // A ring of R step buffers: the loads of step s + R - 1 are issued before
    // step s is computed, so R - 1 steps of K/V rows are in flight per wave.
    const int nsteps = (t1 - t0 + U - 1) / U;
    Buf ring[R];
#pragma unroll
    for (int r = 0; r < R - 1; ++r)
      if (r < nsteps) load(ring[r], t0 + r * U);
    for (int st = 0; st < nsteps; st += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int s = st + r;
        if (s >= nsteps) break;
        if (s + R - 1 < nsteps) load(ring[(r + R - 1) % R], t0 + (s + R - 1) * U);
        compute(ring[r], t0 + s * U);
      }
    }

    if constexpr (STORE && !PREFILL) {
      // fused store: the last step, with the same token boundaries as when
      // streamed, so the result has the same bits as storing first; its older
      // tokens come from the cache, the newest token and its past-the-end copies
      // from k_new / v_new, and the newest token is written to its cache row
      if (t_new >= 0) {
        t1 = t_new + 1;
        Buf fb;
        load(fb, t_fin);
        const int un = t_new - t_fin;
        uint32_t nk[NW], nv[NW];
        const char* kn = (const char*)a.k_new + (int64_t)b * row_bytes + lane_off;
        const char* vn = (const char*)a.v_new + (int64_t)b * row_bytes + lane_off;
        for (int jj = 0; jj < NCH; ++jj) {
          load_words<CH>(&nk[jj * WPC], kn + jj * TL * CH);
          load_words<CH>(&nv[jj * WPC], vn + jj * TL * CH);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (u >= un)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
              fb.k[u][w] = nk[w];
              fb.v[u][w] = nv[w];
            }
        const int64_t r = step_row(t_new);
        for (int jj = 0; jj < NCH; ++jj) {
          store_words<CH>((char*)a.k + r * row_bytes + lane_off + jj * TL * CH, &nk[jj * WPC]);
          store_words<CH>((char*)a.v + r * row_bytes + lane_off + jj * TL * CH, &nv[jj * WPC]);
        }
        compute(fb, t_fin);
      }
    }

    if (nstates == 1) {
      for (int gq = 0; gq < G; ++gq) {
        const float inv = 1.0f / l[gq];
        char* op = (char*)a.out + ((q_row * Hq + g * G + gq) * D) * ELT + c * CH;
        for (int jj = 0; jj < NCH; ++jj) {
          uint32_t w[WPC];
          for (int x = 0; x < WPC; ++x) {
            const int e = (jj * WPC + x) * EPW;
            if constexpr (BF16) {
              w[x] = pack_bf16x2(o[gq][e] * inv, o[gq][e + 1] * inv);
            } else {
              w[x] = __float_as_uint(o[gq][e] * inv);
            }
          }
          store_words<CH>(op + jj * TL * CH, w);
        }
      }
    } else {
      for (int gq = 0; gq < G; ++gq) {
        const int64_t slot = sbase + (int64_t)(g * G + gq) * sstride;
        float* wo = a.ws_o + slot * D;
        for (int jj = 0; jj < NCH; ++jj) {
          const int d0 = (jj * TL + c) * EPC;
          for (int x = 0; x < EPC; ++x) wo[d0 + x] = o[gq][jj * EPC + x];
        }
        if (c == 0) {
          a.ws_ml[slot * 2] = m[gq];
          a.ws_ml[slot * 2 + 1] = l[gq];
        }
      }
    }
  };

  if constexpr (PREFILL) {
    // prefill row i of sequence b (longest rows first): keys 0 .. Lk - Lq + i
    const int b = item % a.num_seqs;
    const int qb = a.cu_seqlens_q[b];
    const int lq = a.cu_seqlens_q[b + 1] - qb;
    const int i = lq - 1 - item / a.num_seqs;
    if (i < 0) return;
    const int k0 = a.cu_seqlens_k[b];
    const int lk = a.cu_seqlens_k[b + 1] - k0;
    segment(b, qb + i, 0, lk - lq + i + 1, k0, 0, 1, 0, 0);
  } else if (a.balance_pieces > 0) {
    // token-balanced: the segments of this wave's range of steps (no range is
    // empty, so the parts of a sequence sit in consecutive waves)
    const int w = item;
    StepScan first;
    long long nmax;
    const long long N = total_steps(a, U, lane, first, nmax);
    const int W = balanced_waves(a.balance_pieces, N, nmax);
    if (w >= W) return;
    const long long s_lo = range_start(w, N, W), s_hi = range_start(w + 1, N, W);
    int b, L, start;
    long long base;
    if (!sequence_of_step(a, U, s_lo, lane, first, b, base, L, start)) return;
    for (long long s = s_lo; s < s_hi && b < a.num_seqs; ++b) {
      if (s > s_lo) {
        L = max(a.context_lens[b], 0);
        start = a.kv_start ? a.kv_start[b] : 0;
      }
      // own keys [start, L): keys below start belong to the group pass
      const long long n = steps_of(L - start, U);
      const long long e = min(s_hi, base + n);
      const int w0 = wave_of_step(base, N, W);
      const int nst = wave_of_step(base + n - 1, N, W) - w0 + 1;
      if (s == base && hg == 0 && lane == 0) {
        a.piece_meta[2 * b] = w0 + b;
        a.piece_meta[2 * b + 1] = nst;
      }
      if (L == 0) {
        write_zeros(b);
      } else {
        // one part and no shared prefix: the output itself; else a state
        segment(b, b, start + (int)((s - base) * U), (int)min((long long)L, start + (e - base) * U), 0, L,
                start > 0 ? 0 : nst, (int64_t)(w + b) * Hq, 1);
      }
      s = e;
      base += n;
    }
  } else {
    // split j of sequence b; keys [0, start) of a sequence with a shared
    // prefix belong to the group pass
    const int b = item % a.num_seqs;
    const int split = item / a.num_seqs;
    const int L = a.context_lens[b];
    const int start = a.kv_start ? a.kv_start[b] : 0;
    if (L == 0) {
      if (split == 0) write_zeros(b);  // an empty context gives zeros
      return;
    }
    const int t0 = start + split * a.split_tokens;
    if (t0 >= L) return;
    // states merged for this row: its splits, plus the group pass's when it has a prefix
    const int nst = (L - start + a.split_tokens - 1) / a.split_tokens + (start > 0 ? 1 : 0);
    const int S = a.ws_stride;
    segment(b, b, t0, min(L, t0 + a.split_tokens), 0, L, nst, (int64_t)b * Hq * S + split, S);
  }
}

__device__ __forceinline__ float readlane_f(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

// One wave merges states lo .. hi-1 of a pair (slot(i) gives their rows):
// M = max_i m_i, den = sum_i 2^(m_i - M) l_i and acc = sum_i 2^(m_i - M) o_i,
// the sums taken one state at a time in index order.  The maxima and sums are
// read 64 states per load (lane k holding state c + k); the partial outputs
// kOB states at a time, the first batch requested together with the first
// maxima, so that up to min(64, kOB) states cost one memory round trip.
template <int D, int kOB, typename Slot>
__device__ __forceinline__ void merge_states(int lo, int hi, const Slot& slot, const float* ml, const float* wo,
                                             int lane, float& M, float& den, float (&acc)[D / 64]) {
  constexpr int EPL = D / 64;
  static_assert(64 % kOB == 0, "output batches must not straddle a 64-state chunk");
  M = kNegInf;
  den = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  if (lo >= hi) return;
  float ov[kOB][EPL];
  auto load_o = [&](int i0) {
#pragma unroll
    for (int k = 0; k < kOB; ++k) {
      if (i0 + k < hi) {  // (uniform) states past the end are not read, nor used
        const int64_t j = slot(i0 + k);
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[k][e] = wo[j * D + e];
      }
    }
  };
  load_o(lo);
  auto load_ml = [&](int c, float& m, float& l) {
    const int i = c + lane;
    m = kNegInf;  // lanes past the end: weight 2^-inf = 0, never read
    l = 0.f;
    if (i < hi) {
      const int64_t j = slot(i);
      m = ml[2 * j];
      l = ml[2 * j + 1];
    }
  };
  float m0, l0;
  load_ml(lo, m0, l0);
  float mx = m0;
  for (int c = lo + 64; c < hi; c += 64) {
    const int i = c + lane;
    if (i < hi) mx = fmaxf(mx, ml[2 * slot(i)]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  M = mx;
  for (int c = lo; c < hi; c += 64) {
    float mc = m0, lc = l0;
    if (c > lo) load_ml(c, mc, lc);
    const float wc = exp2_hw(mc - M);
    const int cend = min(hi, c + 64);
    for (int i0 = c; i0 < cend; i0 += kOB) {
      if (i0 > lo) load_o(i0);
#pragma unroll
      for (int k = 0; k < kOB; ++k) {
        if (i0 + k >= cend) break;
        const float w = readlane_f(wc, i0 + k - c);
        den = fmaf(w, readlane_f(lc, i0 + k - c), den);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, ov[k][e], acc[e]);
      }
    }
  }
}

// Merge the split states of each (sequence, query head): M = max_j m_j,
// w_j = 2^(m_j - M), out = sum_j w_j o_j / sum_j w_j l_j, over the pair's
// states in slot order: its splits (or token-balanced parts), then the group
// pass's chunks of its shared prefix (if any).
//  * WIDE = false (many pairs): one wave per pair (merge_states over all of
//    its states), kReduceWaves pairs per workgroup.
//  * WIDE = true (few pairs, so each may hold hundreds of states): one
//    workgroup per pair; its n states are cut into nw = min(kReduceWaves,
//    ceil(n / 8)) consecutive slices, one per wave, and with nw > 1 the
//    slice results are merged the same way, in slice order.
// With nw = 1 both give the same bits.
constexpr int kReduceWaves = 8;
template <bool BF16, int D, bool WIDE>
__global__ __launch_bounds__(kReduceWaves * 64) void decode_reduce_kernel(RowAttnArgs a) {
  constexpr int EPL = D / 64;  // elements per lane
  const int pair = WIDE ? blockIdx.x : blockIdx.x * kReduceWaves + threadIdx.x / 64;
  const int wv = WIDE ? threadIdx.x / 64 : 0;
  const int lane = threadIdx.x % 64;
  const int Hq = a.num_q_heads;
  if (pair >= a.num_seqs * Hq) return;
  const int b = pair / Hq;
  const int h = pair % Hq;
  const bool balanced = a.balance_pieces > 0;
  int ns, np = 0, first = 0;
  if (balanced) {
    // written by the wave holding the sequence's first step in the split pass
    first = a.piece_meta[2 * b];
    ns = a.piece_meta[2 * b + 1];
    const int start = a.kv_start ? a.kv_start[b] : 0;
    np = start > 0 ? (start + a.prefix_chunk - 1) / a.prefix_chunk : 0;
  } else {
    const int L = a.context_lens[b];
    const int start = a.kv_start ? a.kv_start[b] : 0;
    ns = (L - start + a.split_tokens - 1) / a.split_tokens;
    np = start > 0 ? (start + a.prefix_chunk - 1) / a.prefix_chunk : 0;
  }
  if (np == 0 && ns <= 1) return;
  const int S = a.ws_stride;
  // state of the i-th merged term: parts first .. first + ns - 1 of the
  // sequence (token-balanced), then its prefix chunks in their own region;
  // else the pair's splits 0 .. ns-1, then its prefix chunks at num_splits ..
  auto slot = [&](int i) -> int64_t {
    if (balanced)
      return i < ns ? (int64_t)(first + i) * Hq + h : a.prefix_slot0 + (int64_t)pair * a.prefix_states + (i - ns);
    return (int64_t)pair * S + (i < ns ? i : a.num_splits + (i - ns));
  };
  const int n = ns + np;
  const int nw = WIDE ? min(kReduceWaves, (n + 7) / 8) : 1;
  const int per = (n + nw - 1) / nw;
  const int lo = min(n, wv * per), hi = min(n, lo + per);
  float M, den, acc[EPL];
  merge_states<D, 16>(lo, hi, slot, a.ws_ml, a.ws_o + lane * EPL, lane, M, den, acc);
  if (WIDE && nw > 1) {
    // merge the slices' (M, den, acc) in slice order (nw is the same for the
    // whole workgroup, so every wave reaches the barrier)
    __shared__ float part_m[kReduceWaves], part_l[kReduceWaves];
    __shared__ float part_o[kReduceWaves][D];
    if (wv < nw) {
      if (lane == 0) {
        part_m[wv] = M;
        part_l[wv] = den;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) part_o[wv][lane * EPL + e] = acc[e];
    }
    __syncthreads();
    if (wv != 0) return;
    M = kNegInf;
    for (int j = 0; j < nw; ++j) M = fmaxf(M, part_m[j]);
    den = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int j = 0; j < nw; ++j) {
      const float w = exp2_hw(part_m[j] - M);
      den = fmaf(w, part_l[j], den);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, part_o[j][lane * EPL + e], acc[e]);
    }
  } else if (wv != 0) {
    return;
  }
  const float inv = 1.0f / den;
  if constexpr (BF16) {
    uint16_t* op = (uint16_t*)a.out + (int64_t)pair * D + lane * EPL;
    if constexpr (EPL == 2) {
      *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      op[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
    }
  } else {
    float* op = (float*)a.out + (int64_t)pair * D + lane * EPL;
    for (int e = 0; e < EPL; ++e) op[e] = acc[e] * inv;
  }
}

}  // namespace pkv
