// Rotary embedding of q and k fused with the paged cache write of k and v.
//
// The rotation is the RoFormer one: dimension pair j of every head of token i
// turns by positions[i] * theta^(-2j/D), the pair being (j, j + D/2)
// ("rotate-half") or (2j, 2j + 1) ("interleaved").  q is rotated in place; the
// rotated k row and the v row go to slot_mapping[i] of the caches (a negative
// slot skips the cache write, not the rotation of q).
//
// A workgroup of 256 threads takes one token.  Its work is a list of tasks:
// the q tasks, then the k tasks, then (when the token has a slot) the 16-byte
// chunks of its v row.  A q or k task is 8 pairs of one head: two 8-element
// runs, (8c .. 8c+7, D/2 + 8c .. D/2 + 8c + 7) in rotate-half layout or
// 16c .. 16c + 15 interleaved, so consecutive lanes cover a head row.  Every
// thread issues the loads of its first two tasks before anything else; the
// token's D/2 angles are meanwhile formed and reduced modulo 2 pi in fp64 (an angle
// reaches position * 1 rad, far beyond where an fp32 product keeps its
// fraction) and turned into (cos, sin) in LDS, shared by all heads.  So a
// token costs one memory round trip (more only past 512 tasks, e.g. 64 query
// heads of 128 dims).
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

// 8 elements of storage type T in 16-byte units.
template <typename T>
struct Run8 {
  static constexpr int kVecs = sizeof(T) * 8 / 16;  // bf16: 1, fp32: 2
  uint4 w[kVecs];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) w[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ void store(T* p) const {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) reinterpret_cast<uint4*>(p)[i] = w[i];
  }
  __device__ __forceinline__ float get(int t) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t x = (&w[0].x)[t >> 1];
      return (t & 1) ? bf16_hi(x) : bf16_lo(x);
    } else {
      return __uint_as_float((&w[0].x)[t]);
    }
  }
  // sets elements t and t + 1 (t even)
  __device__ __forceinline__ void set2(int t, float a, float b) {
    if constexpr (sizeof(T) == 2) {
      (&w[0].x)[t >> 1] = pack_bf16x2(a, b);
    } else {
      (&w[0].x)[t] = __float_as_uint(a);
      (&w[0].x)[t + 1] = __float_as_uint(b);
    }
  }
};

// Rotates the 8 pairs of one task; cs holds (cos, sin) of the token's pairs, f0 = 8c.
template <typename T, bool INTERLEAVED>
__device__ __forceinline__ void rotate(Run8<T>& a, Run8<T>& b, const float2* cs, int f0) {
  if constexpr (INTERLEAVED) {
    // pairs (a0,a1) (a2,a3) (a4,a5) (a6,a7) (b0,b1) ... are pairs f0 .. f0 + 7
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      Run8<T>& r = half ? b : a;
      float o[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float2 e = cs[f0 + 4 * half + t];
        const float x = r.get(2 * t), y = r.get(2 * t + 1);
        o[2 * t] = x * e.x - y * e.y;
        o[2 * t + 1] = x * e.y + y * e.x;
      }
#pragma unroll
      for (int t = 0; t < 8; t += 2) r.set2(t, o[t], o[t + 1]);
    }
  } else {
    // pair f0 + t is (a_t, b_t)
    float oa[8], ob[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 e = cs[f0 + t];
      const float x = a.get(t), y = b.get(t);
      oa[t] = x * e.x - y * e.y;
      ob[t] = x * e.y + y * e.x;
    }
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      a.set2(t, oa[t], oa[t + 1]);
      b.set2(t, ob[t], ob[t + 1]);
    }
  }
}

// Element offsets, inside a head row, of the two runs of task chunk c.
template <int D, bool INTERLEAVED>
__device__ __forceinline__ int2 run_offsets(int c) {
  if constexpr (INTERLEAVED) return make_int2(16 * c, 16 * c + 8);
  return make_int2(8 * c, D / 2 + 8 * c);
}

// One task of a token: what it is and where it reads and writes (element
// offsets from the bases of its kind: q for q, k / k_cache for k, v / v_cache
// for v).
template <int D>
struct RopeTask {
  int kind;     // 0 q, 1 k, 2 v
  int c;        // chunk within the head (q, k)
  int64_t src;  // element offset of the head row (q, k) or of the 16-byte chunk (v)
  int64_t dst;
};

template <typename T, int D>
__device__ __forceinline__ RopeTask<D> rope_task(int Hq, int Hkv, int64_t token, int32_t slot, int u) {
  constexpr int CH = D / 16;
  const int nq = Hq * CH, nk = Hkv * CH;
  const int64_t row = (int64_t)Hkv * D;
  RopeTask<D> t;
  if (u < nq) {
    t.kind = 0;
    t.c = u % CH;
    t.src = t.dst = (token * Hq + u / CH) * D;
  } else if (u < nq + nk) {
    t.kind = 1;
    t.c = (u - nq) % CH;
    t.src = token * row + ((u - nq) / CH) * D;
    t.dst = (int64_t)slot * row + ((u - nq) / CH) * D;
  } else {
    t.kind = 2;
    t.c = 0;
    const int e = (u - nq - nk) * (16 / (int)sizeof(T));
    t.src = token * row + e;
    t.dst = (int64_t)slot * row + e;
  }
  return t;
}

// Pointers of the three kinds of task: sources and destinations.
template <typename T>
struct RopePtrs {
  T* q;
  const T* k;
  const T* v;
  T* k_cache;
  T* v_cache;
};

template <typename T, int D, bool INTERLEAVED>
__device__ __forceinline__ void task_load(const RopePtrs<T>& p, const RopeTask<D>& t, Run8<T>& ra, Run8<T>& rb) {
  const T* base = t.kind == 0 ? p.q : t.kind == 1 ? p.k : p.v;
  if (t.kind == 2) {
    ra.w[0] = *reinterpret_cast<const uint4*>(base + t.src);
  } else {
    const int2 off = run_offsets<D, INTERLEAVED>(t.c);
    ra.load(base + t.src + off.x);
    rb.load(base + t.src + off.y);
  }
}

template <typename T, int D, bool INTERLEAVED>
__device__ __forceinline__ void task_finish(const RopePtrs<T>& p, const RopeTask<D>& t, Run8<T>& ra, Run8<T>& rb,
                                            const float2* cs) {
  T* base = t.kind == 0 ? p.q : t.kind == 1 ? p.k_cache : p.v_cache;
  if (t.kind == 2) {
    *reinterpret_cast<uint4*>(base + t.dst) = ra.w[0];
  } else {
    rotate<T, INTERLEAVED>(ra, rb, cs, 8 * t.c);
    const int2 off = run_offsets<D, INTERLEAVED>(t.c);
    ra.store(base + t.dst + off.x);
    rb.store(base + t.dst + off.y);
  }
}

template <typename T, int D, bool INTERLEAVED>
__global__ __launch_bounds__(256) void rope_kv_store_kernel(RopeStoreArgs a) {
  constexpr int CH = D / 16;  // q / k tasks per head
  __shared__ float2 cs[D / 2];
  const int64_t token = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t slot = a.slot_mapping[token];
  const int32_t pos = a.positions[token];
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const RopePtrs<T> p{static_cast<T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                      static_cast<T*>(a.k_cache), static_cast<T*>(a.v_cache)};
  const int nq = Hq * CH;
  // with no slot only q is rotated
  const int ntask = slot < 0 ? nq : nq + Hkv * CH + (int)((int64_t)Hkv * D * sizeof(T) / 16);

  Run8<T> r0a, r0b, r1a, r1b;
  const bool has0 = tid < ntask, has1 = tid + 256 < ntask;
  const RopeTask<D> t0 = rope_task<T, D>(Hq, Hkv, token, slot, tid);
  const RopeTask<D> t1 = rope_task<T, D>(Hq, Hkv, token, slot, tid + 256);
  if (has0) task_load<T, D, INTERLEAVED>(p, t0, r0a, r0b);
  if (has1) task_load<T, D, INTERLEAVED>(p, t1, r1a, r1b);

  if (tid < D / 2) {
    // angle = position * theta^(-2j/D), reduced to [-pi, pi] in fp64
    const double ang = (double)pos * exp2(-2.0 * tid / D * a.log2_theta);
    const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cn;
    sincosf((float)r, &sn, &cn);
    cs[tid] = make_float2(cn, sn);
  }
  __syncthreads();

  if (has0) task_finish<T, D, INTERLEAVED>(p, t0, r0a, r0b, cs);
  if (has1) task_finish<T, D, INTERLEAVED>(p, t1, r1a, r1b, cs);
  for (int u = tid + 512; u < ntask; u += 256) {
    const RopeTask<D> t = rope_task<T, D>(Hq, Hkv, token, slot, u);
    Run8<T> ra, rb;
    task_load<T, D, INTERLEAVED>(p, t, ra, rb);
    task_finish<T, D, INTERLEAVED>(p, t, ra, rb, cs);
  }
}

}  // namespace

hipError_t launch_rope_kv_store(const RopeStoreArgs& a, int32_t dtype, int32_t head_dim, bool interleaved,
                                hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (a.num_tokens > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)a.num_tokens), block(256);
#define PKV_ROPE_CASE(T, DT, DD, IL)                                                                   \
  if (dtype == DT && head_dim == DD && interleaved == IL) {                                            \
    hipLaunchKernelGGL((rope_kv_store_kernel<T, DD, IL>), grid, block, 0, stream, a);                 \
    return hipGetLastError();                                                                         \
  }
  PKV_ROPE_CASE(uint16_t, kBF16, 128, false)
  PKV_ROPE_CASE(uint16_t, kBF16, 128, true)
  PKV_ROPE_CASE(uint16_t, kBF16, 64, false)
  PKV_ROPE_CASE(uint16_t, kBF16, 64, true)
  PKV_ROPE_CASE(float, kF32, 128, false)
  PKV_ROPE_CASE(float, kF32, 128, true)
  PKV_ROPE_CASE(float, kF32, 64, false)
  PKV_ROPE_CASE(float, kF32, 64, true)
#undef PKV_ROPE_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
