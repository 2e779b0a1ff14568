// Row attention on the vector units: one wave = one query row of every head
// of HPW KV heads, streaming that row's keys through the block table.
//
//  * Decode: a row is sequence b's new token; its context is cut into splits
//    of split_tokens keys, one wave per (sequence, KV-head group, split).
//    Splits write an unnormalised softmax state that decode_reduce merges.
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

// Wave-wide sum and inclusive prefix sum (64 lanes).
__device__ __forceinline__ long long wave_sum_i64(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Token-balanced decode: the piece a wave works on (see RowAttnArgs).  Every
// wave derives the same piece boundaries from context_lens: the total (one
// pass over the lengths), then each sequence's piece count and a running
// prefix sum until the sequence holding piece w.  Returns false past the
// last piece.
__device__ __forceinline__ bool balanced_piece(const RowAttnArgs& a, int w, int lane, int& b, int& j, int& off_b,
                                               int& n_b, int& len_b) {
  const int B = a.num_seqs;
  long long tot = 0;
  for (int i = lane; i < B; i += 64) tot += max(a.context_lens[i], 0);
  tot = wave_sum_i64(tot);
  const long long room = max((long long)a.balance_pieces - B, 1LL);
  const long long per = (tot + room - 1) / room;
  const int T = (int)min(max(64LL, (per + 63) / 64 * 64), (long long)0x40000000);
  int base = 0;
  for (int i0 = 0; i0 < B; i0 += 64) {
    const int i = i0 + lane;
    const int L = i < B ? max(a.context_lens[i], 0) : 0;
    const int n = i < B ? max(1, (L + T - 1) / T) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    const int off = base + incl - n;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(i < B && off <= w && w < off + n);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      b = i0 + src;
      off_b = __builtin_amdgcn_readlane(off, src);
      n_b = __builtin_amdgcn_readlane(n, src);
      const int Lb = __builtin_amdgcn_readlane(L, src);
      len_b = ((Lb + n_b - 1) / n_b + 63) / 64 * 64;
      j = w - off_b;
      return true;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
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
  // decode pieces: split j_or_row of sequence b, fixed length or token-balanced
  const bool balanced = !PREFILL && a.balance_pieces > 0;
  int b, j_or_row, off_b = 0, n_bal = 1, len_b = 0;
  if (balanced) {
    if (!balanced_piece(a, item, lane, b, j_or_row, off_b, n_bal, len_b)) return;
  } else {
    b = item % a.num_seqs;
    j_or_row = item / a.num_seqs;
  }
  const int g = hg * HPW + hl;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int64_t row_bytes = (int64_t)Hkv * D * ELT;

  // This wave's query row, its key range [t0, t1), and the split index.
  int64_t q_row;
  int t0, t1, split = 0, nsplit_b = 1, k0 = 0;
  int t_new = -1;  // fused store: position of the newest token if this wave's range holds it
  int t_fin = -1;  // fused store: first token of the step that holds it
  if constexpr (PREFILL) {
    const int qb = a.cu_seqlens_q[b];
    const int lq = a.cu_seqlens_q[b + 1] - qb;
    const int i = lq - 1 - j_or_row;  // longest rows first
    if (i < 0) return;
    k0 = a.cu_seqlens_k[b];
    const int lk = a.cu_seqlens_k[b + 1] - k0;
    q_row = qb + i;
    t0 = 0;
    t1 = lk - lq + i + 1;
  } else {
    // keys [0, start) of a sequence with a shared prefix belong to the group pass
    const int L = a.context_lens[b];
    const int start = a.kv_start ? a.kv_start[b] : 0;
    split = j_or_row;
    q_row = b;
    const int piece = balanced ? len_b : a.split_tokens;
    t0 = start + split * piece;
    if (L == 0) {
      if (split == 0) {  // an empty context gives zeros
        for (int gq = 0; gq < G; ++gq) {
          char* op = (char*)a.out + ((q_row * Hq + g * G + gq) * D) * ELT + c * CH;
          uint32_t z[WPC] = {};
          for (int jj = 0; jj < NCH; ++jj) store_words<CH>(op + jj * TL * CH, z);
        }
      }
      return;
    }
    if (t0 >= L) return;
    t1 = min(L, t0 + piece);
    if (STORE && t1 == L) {
      // the step holding the newest token is taken out of the streaming loop
      // and done after it, with that token read from k_new / v_new
      t_new = L - 1;
      t_fin = t0 + (t_new - t0) / U * U;
      t1 = t_fin;
    }
    // states merged for this row: its splits, plus the group pass's when it has a prefix
    nsplit_b = balanced ? n_bal : (L - start + a.split_tokens - 1) / a.split_tokens + (start > 0 ? 1 : 0);
    if (balanced && split == 0 && hg == 0 && lane == 0) {
      a.piece_meta[2 * b] = off_b;
      a.piece_meta[2 * b + 1] = n_bal;
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
  static_assert(!BF16 || U % 2 == 0, "bf16 steps pair tokens");
  const uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
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

  if (nsplit_b == 1) {
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
    const int S = a.ws_stride;
    for (int gq = 0; gq < G; ++gq) {
      const int64_t slot = balanced ? (int64_t)(off_b + split) * Hq + g * G + gq
                                    : ((int64_t)b * Hq + g * G + gq) * S + split;
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
}

// Merge the split states of each (sequence, query head): M = max_j m_j,
// w_j = 2^(m_j - M), out = sum_j w_j o_j / sum_j w_j l_j.  One wave per pair,
// states merged in slot order: the pair's splits, then the group pass's
// chunks of its shared prefix (if any).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(RowAttnArgs a) {
  constexpr int EPL = D / 64;  // elements per lane
  const int pair = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int Hq = a.num_q_heads;
  if (pair >= a.num_seqs * Hq) return;
  const int b = pair / Hq;
  const int h = pair % Hq;
  const bool balanced = a.balance_pieces > 0;
  int ns, np = 0, first = 0;
  if (balanced) {
    // written by the first piece of the sequence in the split pass
    first = a.piece_meta[2 * b];
    ns = a.piece_meta[2 * b + 1];
  } else {
    const int L = a.context_lens[b];
    const int start = a.kv_start ? a.kv_start[b] : 0;
    ns = (L - start + a.split_tokens - 1) / a.split_tokens;
    np = start > 0 ? (start + a.prefix_chunk - 1) / a.prefix_chunk : 0;
  }
  if (np == 0 && ns <= 1) return;
  const int S = a.ws_stride;
  const float* ml = a.ws_ml;
  const float* wo = a.ws_o + lane * EPL;
  // state of the i-th merged term: balanced pieces first .. first + ns - 1 of
  // the sequence; else the pair's splits 0 .. ns-1, then its prefix chunks at
  // num_splits ..
  auto slot = [&](int i) -> int64_t {
    if (balanced) return (int64_t)(first + i) * Hq + h;
    return (int64_t)pair * S + (i < ns ? i : a.num_splits + (i - ns));
  };
  // States are read kBatch at a time, so that their loads are in flight
  // together (the first batch's with the maxima of the rest: one memory round
  // trip for up to kBatch states); they are combined one by one in slot order.
  constexpr int kBatch = 8;
  const int n = ns + np;
  float mv[kBatch], lv[kBatch], ov[kBatch][EPL];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t j = slot(min(i0 + k, n - 1));  // past the end: the last state again, unused
      mv[k] = ml[2 * j];
      lv[k] = ml[2 * j + 1];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ov[k][e] = wo[j * D + e];
    }
  };
  load_batch(0);
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < kBatch; ++k) M = fmaxf(M, mv[k]);  // repeats leave the max alone
  for (int i0 = kBatch; i0 < n; i0 += kBatch) {
    float mx[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mx[k] = ml[2 * slot(min(i0 + k, n - 1))];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) M = fmaxf(M, mx[k]);
  }
  float den = 0.f, acc[EPL] = {};
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    if (i0 > 0) load_batch(i0);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (i0 + k >= n) break;
      const float w = exp2_hw(mv[k] - M);
      den = fmaf(w, lv[k], den);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, ov[k][e], acc[e]);
    }
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
