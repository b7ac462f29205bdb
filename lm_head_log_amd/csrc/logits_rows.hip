// logits_rows.hip - log-prob / entropy from logits that already exist in
// memory, for MI355X (gfx950): the entry points lmhead_logits_fwd and
// lmhead_logits_bwd declared in include/lmhead.h.
//
// This is the contract of twinkle PR #283, section 1 (selective_log_softmax):
// the caller holds the [N, V] logits (bf16 or fp32); per row the op returns
// the target's log-probability and the entropy in fp32 and, in backward,
// recomputes the softmax from the logits instead of keeping it. The pages'
// version walks the rows in chunks to bound its temporaries; these kernels
// keep no temporaries at all (each row is streamed once per pass), so the
// chunking has nothing left to bound.
//
// One workgroup per row. The work is a stream over the row with a few VALU
// operations per element, so the bound is HBM bandwidth: the forward reads
// the logits once, the backward reads them once more and writes the gradient.
// Loads are 16 bytes per lane, consecutive lanes on consecutive 16-byte
// chunks (each wave reads 1 KiB of a row per instruction).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/lmhead.h"
#include "launch.h"

#define LMH_API extern "C" __attribute__((visibility("default")))

namespace lmh_rows {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A -inf logit (a token the model rules out) counts as probability 0: logits
// and their scaled differences are clamped to this finite value, whose
// exponential is 0 next to any real maximum while 0 * value stays finite.
constexpr float kFloor = -1e30f;
constexpr int kThreads = 256;
// One workgroup per row; a launch may hold at most 2^32 work-items, so rows
// go in launches of at most 2^22 workgroups.
constexpr int64_t kRowsPerLaunch = int64_t(1) << 22;
constexpr int kUnroll = 4;

__device__ __forceinline__ float load_one(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
__device__ __forceinline__ float load_one(const float* p) { return *p; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Elements per 16-byte vector; rows are streamed once, so the vector
// accesses are non-temporal.
template <class T>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8]) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8]) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2_t h = {(__bf16)x[2 * k], (__bf16)x[2 * k + 1]};  // round to nearest even
      w[k] = __builtin_bit_cast(uint32_t, h);
    }
    const u32x4_t v = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
  }
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    x[0] = v[0];
    x[1] = v[1];
    x[2] = v[2];
    x[3] = v[3];
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
    const f32x4_t v = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
  }
};

__device__ __forceinline__ void store_one(uint16_t* p, float x) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ void store_one(float* p, float x) { *p = x; }

// Online statistics in base-2 units over a set S of logits z, y = z log2 e:
// m = max y, s = sum 2^(y - m), b = sum 2^(y - m) (y - m).
struct Stats {
  float m = -INFINITY, s = 0.f, b = 0.f;

  // Adds logits whose maximum is cz.
  template <int K>
  __device__ __forceinline__ void add(const float (&z)[K], float cz) {
    const float cm = fmaxf(cz * kLog2e, kFloor);
    if (cm > m) {
      // rescale to the new maximum: b' = a (b + (m - m') s), s' = a s
      if (m != -INFINITY) {
        const float d = m - cm;
        const float a = exp2f(d);
        b = a * fmaf(d, s, b);
        s *= a;
      }
      m = cm;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      // d <= 0: the hardware exp2 (results below 2^-126 flush to 0, which
      // next to the maximum's 1 changes nothing)
      const float d = fmaxf(fmaf(z[k], kLog2e, -m), kFloor);
      const float e = __builtin_amdgcn_exp2f(d);
      s += e;
      b = fmaf(e, d, b);
    }
  }

  // Merges another partial (two partials combine exactly up to rounding).
  __device__ __forceinline__ void merge(float m2, float s2, float b2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    float a1 = 0.f, a2 = 0.f, t1 = 0.f, t2 = 0.f;
    if (m != -INFINITY) {
      const float d = m - mn;
      a1 = exp2f(d);
      t1 = a1 * fmaf(d, s, b);
      a1 *= s;
    }
    if (m2 != -INFINITY) {
      const float d = m2 - mn;
      a2 = exp2f(d);
      t2 = a2 * fmaf(d, s2, b2);
      a2 *= s2;
    }
    m = mn;
    s = a1 + a2;
    b = t1 + t2;
  }
};

// Elements of the row before the first 16-byte boundary.
template <class T>
__device__ __forceinline__ int64_t head_len(const T* row, int64_t V) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(row);
  const int64_t h = (int64_t)(((16 - (a & 15)) & 15) / sizeof(T));
  return h < V ? h : V;
}

template <class T>
__global__ __launch_bounds__(kThreads) void k_logits_fwd(const T* __restrict__ logits, int64_t r0,
                                                          int64_t V,
                                                          const int32_t* __restrict__ targets,
                                                          const uint8_t* __restrict__ keep,
                                                          float* __restrict__ logp,
                                                          float* __restrict__ entropy,
                                                          float* __restrict__ stats) {
  __shared__ float red[3][kThreads / 64];
  const int64_t i = r0 + blockIdx.x;
  const int tid = threadIdx.x;
  if (keep && keep[i] == 0) {
    if (tid == 0) {
      logp[i] = 0.f;
      if (entropy) entropy[i] = 0.f;
      stats[2 * i] = 0.f;
      stats[2 * i + 1] = 0.f;
    }
    return;
  }
  const T* row = logits + i * V;
  constexpr int K = Vec<T>::n;
  Stats st;
  const int64_t h = head_len(row, V);
  const int64_t nv = (V - h) / K;  // whole vectors after the head
  // head and tail elements one at a time
  for (int64_t v = tid; v < h; v += kThreads) {
    const float z[1] = {load_one(row + v)};
    st.add(z, z[0]);
  }
  for (int64_t v = h + nv * K + tid; v < V; v += kThreads) {
    const float z[1] = {load_one(row + v)};
    st.add(z, z[0]);
  }
  const T* body = row + h;
  // kUnroll vectors in flight per lane: with one, the loads a CU keeps in
  // flight cannot cover the memory latency at full bandwidth
  int64_t c = tid;
  for (; c + (kUnroll - 1) * kThreads < nv; c += kUnroll * kThreads) {
    float z[kUnroll][K];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Vec<T>::load(body + (c + u * kThreads) * K, z[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float cz = z[u][0];
#pragma unroll
      for (int k = 1; k < K; ++k) cz = fmaxf(cz, z[u][k]);
      st.add(z[u], cz);
    }
  }
  for (; c < nv; c += kThreads) {
    float z[K];
    Vec<T>::load(body + c * K, z);
    float cz = z[0];
#pragma unroll
    for (int k = 1; k < K; ++k) cz = fmaxf(cz, z[k]);
    st.add(z, cz);
  }
  // wave then workgroup reduction, in a fixed order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    st.merge(__shfl_xor(st.m, off), __shfl_xor(st.s, off), __shfl_xor(st.b, off));
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][wave] = st.m;
    red[1][wave] = st.s;
    red[2][wave] = st.b;
  }
  __syncthreads();
  if (tid == 0) {
    Stats t;
    for (int w = 0; w < kThreads / 64; ++w) t.merge(red[0][w], red[1][w], red[2][w]);
    const float l2s = log2f(t.s);
    const float lse = (t.m + l2s) * kLn2;
    const float ent = (l2s - t.b / t.s) * kLn2;
    const int tt = targets[i];
    const float lp = (tt >= 0 && tt < V) ? load_one(row + tt) - lse : __builtin_nanf("");
    logp[i] = lp;
    if (entropy) entropy[i] = ent;
    stats[2 * i] = lse;
    stats[2 * i + 1] = ent;
  }
}

// dz = g_lp (onehot - p) - g_H p (ln p + H), p = e^(z - LSE), written in the
// logits' precision (bf16 rounds to nearest even); skipped rows get +0.0.
template <class T>
__global__ __launch_bounds__(kThreads) void k_logits_bwd(
    const T* __restrict__ logits, int64_t r0, int64_t V, const int32_t* __restrict__ targets,
    const uint8_t* __restrict__ keep, const float* __restrict__ stats,
    const float* __restrict__ g_lp, const float* __restrict__ g_h, T* __restrict__ grad) {
  const int64_t i = r0 + blockIdx.x;
  const int tid = threadIdx.x;
  const T* row = logits + i * V;
  T* out = grad + i * V;
  constexpr int K = Vec<T>::n;
  const int64_t h = head_len(row, V);
  const int64_t nv = (V - h) / K;
  if (keep && keep[i] == 0) {
    const float zero[K] = {};
    for (int64_t v = tid; v < h; v += kThreads) store_one(out + v, 0.f);
    for (int64_t v = h + nv * K + tid; v < V; v += kThreads) store_one(out + v, 0.f);
    for (int64_t c = tid; c < nv; c += kThreads) Vec<T>::store(out + h + c * K, zero);
    return;
  }
  // dz = p (ca' + cb z) + g_lp [v = t], p = 2^(z log2 e - LSE log2 e),
  // ca' = ca - cb LSE, ca = -(g_lp + g_H H), cb = -g_H
  const float lse = stats[2 * i], ent = stats[2 * i + 1];
  const float gl = g_lp[i];
  const float gh = g_h ? g_h[i] : 0.f;
  const float cb = -gh;
  const float ca = -(gl + gh * ent) - cb * lse;
  const float l2 = lse * kLog2e;
  const int64_t tt = targets[i];
  auto dz = [&](float z) {
    const float zc = fmaxf(z, kFloor);
    const float p = __builtin_amdgcn_exp2f(fmaf(zc, kLog2e, -l2));
    return p * fmaf(cb, zc, ca);
  };
  for (int64_t v = tid; v < h; v += kThreads)
    store_one(out + v, dz(load_one(row + v)) + (v == tt ? gl : 0.f));
  for (int64_t v = h + nv * K + tid; v < V; v += kThreads)
    store_one(out + v, dz(load_one(row + v)) + (v == tt ? gl : 0.f));
  const T* body = row + h;
  T* obody = out + h;
  auto finish = [&](int64_t c, float (&z)[K]) {
    float d[K];
#pragma unroll
    for (int k = 0; k < K; ++k) d[k] = dz(z[k]);
    const int64_t local = tt - (h + c * K);
    if (local >= 0 && local < K) {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (k == local) d[k] += gl;
    }
    Vec<T>::store(obody + c * K, d);
  };
  int64_t c = tid;
  for (; c + (kUnroll - 1) * kThreads < nv; c += kUnroll * kThreads) {
    float z[kUnroll][K];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Vec<T>::load(body + (c + u * kThreads) * K, z[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) finish(c + u * kThreads, z[u]);
  }
  for (; c < nv; c += kThreads) {
    float z[K];
    Vec<T>::load(body + c * K, z);
    finish(c, z);
  }
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

static int check_rows(const void* logits, int dtype, int64_t N, int64_t V) {
  if (N < 0 || V <= 0) return LMHEAD_ERR_INVALID_ARG;
  if (dtype != LMHEAD_DTYPE_BF16 && dtype != LMHEAD_DTYPE_F32) return LMHEAD_ERR_UNSUPPORTED;
  if (N > (int64_t(1) << 31) - 1 || V > (int64_t(1) << 31) - 1) return LMHEAD_ERR_UNSUPPORTED;
  if (N > 0 && !logits) return LMHEAD_ERR_INVALID_ARG;
  if (dtype == LMHEAD_DTYPE_F32 && !aligned4(logits)) return LMHEAD_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(logits) & 1) != 0) return LMHEAD_ERR_INVALID_ARG;
  return LMHEAD_OK;
}

}  // namespace lmh_rows

using namespace lmh_rows;

LMH_API int lmhead_logits_fwd(const void* logits, int dtype, int64_t N, int64_t V,
                              const int32_t* targets, const uint8_t* keep_mask,
                              int return_entropy, float* logp, float* entropy,
                              float* saved_stats, void* stream) {
  int st = check_rows(logits, dtype, N, V);
  if (st != LMHEAD_OK) return st;
  if (N > 0 && (!targets || !logp || !saved_stats)) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (return_entropy != 0) != (entropy != nullptr)) return LMHEAD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < N; r0 += kRowsPerLaunch) {
    const dim3 grid((unsigned)std::min<int64_t>(N - r0, kRowsPerLaunch));
    const hipError_t e =
        dtype == LMHEAD_DTYPE_BF16
            ? lmh_launch::launch_kernel(k_logits_fwd<uint16_t>, grid, dim3(kThreads), s,
                                        static_cast<const uint16_t*>(logits), r0, V, targets,
                                        keep_mask, logp, entropy, saved_stats)
            : lmh_launch::launch_kernel(k_logits_fwd<float>, grid, dim3(kThreads), s,
                                        static_cast<const float*>(logits), r0, V, targets,
                                        keep_mask, logp, entropy, saved_stats);
    if (e != hipSuccess) return LMHEAD_ERR_HIP;
  }
  return LMHEAD_OK;
}

LMH_API int lmhead_logits_bwd(const void* logits, int dtype, int64_t N, int64_t V,
                              const int32_t* targets, const uint8_t* keep_mask,
                              const float* saved_stats, const float* grad_logp,
                              const float* grad_entropy, int entropy_requires_grad,
                              void* grad_logits, void* stream) {
  int st = check_rows(logits, dtype, N, V);
  if (st != LMHEAD_OK) return st;
  if (N > 0 && (!targets || !saved_stats || !grad_logp || !grad_logits))
    return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (entropy_requires_grad != 0) != (grad_entropy != nullptr))
    return LMHEAD_ERR_INVALID_ARG;
  // the gradient has the logits' layout, so the same element alignment
  if ((reinterpret_cast<uintptr_t>(grad_logits) & 15) !=
      (reinterpret_cast<uintptr_t>(logits) & 15))
    return LMHEAD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* gh = entropy_requires_grad ? grad_entropy : nullptr;
  for (int64_t r0 = 0; r0 < N; r0 += kRowsPerLaunch) {
    const dim3 grid((unsigned)std::min<int64_t>(N - r0, kRowsPerLaunch));
    const hipError_t e =
        dtype == LMHEAD_DTYPE_BF16
            ? lmh_launch::launch_kernel(k_logits_bwd<uint16_t>, grid, dim3(kThreads), s,
                                        static_cast<const uint16_t*>(logits), r0, V, targets,
                                        keep_mask, saved_stats, grad_logp, gh,
                                        static_cast<uint16_t*>(grad_logits))
            : lmh_launch::launch_kernel(k_logits_bwd<float>, grid, dim3(kThreads), s,
                                        static_cast<const float*>(logits), r0, V, targets,
                                        keep_mask, saved_stats, grad_logp, gh,
                                        static_cast<float*>(grad_logits));
    if (e != hipSuccess) return LMHEAD_ERR_HIP;
  }
  return LMHEAD_OK;
}
