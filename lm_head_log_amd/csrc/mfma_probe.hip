// mfma_probe.hip - benchmark-only measurement of the MFMA ceiling the GEMM
// kernels run against on the device at hand.
//
// The GEMMs of the op issue v_mfma_f32_16x16x32_bf16 in 8 x 8 blocks per
// wave (the engine's in-place form), four waves per CU, one workgroup per CU.
// This kernel issues exactly that step with every operand already in
// registers: no loads, no LDS, no barriers, no epilogue. Its rate is therefore the most the GEMM engine could
// reach at the clock the chip holds under that MFMA load. The chip lowers its
// clock with the power the matrix cores draw, and that power depends on how
// often operand bits change, so the operands can be taken from the caller's
// own tensors (the same bits the GEMMs multiply) or be all zero (the least
// switching activity). The shader clock is read with s_memtime at the start
// and end of each workgroup's loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/lmhead.h"
#include "gemm_core.h"
#include "launch.h"

#define LMH_API extern "C" __attribute__((visibility("default")))

namespace lmh {
namespace {

constexpr int kProbeSets = 2;  // fragment sets cycled through, one per k step
constexpr int kProbeWavesPerGroup = kThreads / 64;
constexpr int64_t kProbeMaxIters = int64_t(1) << 24;

// Eight consecutive bf16 values of `p` (16-byte aligned) at group `slot` of
// `groups` 8-value groups; zeros when p is null.
__device__ __forceinline__ bf16x8_t probe_frag(const uint16_t* __restrict__ p, uint32_t groups,
                                               uint32_t slot) {
  if (p == nullptr) {
    const bf16x8_t z = {};
    return z;
  }
  return *reinterpret_cast<const bf16x8_t*>(p + (size_t)(slot % groups) * 8);
}

__global__ __launch_bounds__(kThreads, 1) void k_mfma_probe(
    const uint16_t* __restrict__ a, uint32_t a_groups, const uint16_t* __restrict__ b,
    uint32_t b_groups, int iters, unsigned long long* __restrict__ cycles,
    float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t gw = blockIdx.x * kProbeWavesPerGroup + (threadIdx.x >> 6);
  Frags f[kProbeSets];
#pragma unroll
  for (int s = 0; s < kProbeSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // a distinct 16-byte piece of each source per (wave, set, fragment, lane)
      const uint32_t slot = ((gw * kProbeSets + s) * 8 + i) * 64 + lane;
      f[s].a[i] = probe_frag(a, a_groups, slot);
      f[s].b[i] = probe_frag(b, b_groups, slot);
    }
  Acc acc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  acc_pin(acc);

  __syncthreads();  // the fragments of every wave are in registers
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kProbeSets; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int j = mfma_col(i * 8 + c);  // the engine's order
          mfma16(acc[i][j], f[s].a[i], f[s].b[j]);
        }
  }
  acc_fence(acc);
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);

  // keep every product live: one sum per thread
  float x = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) x += acc[i][j][r];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

int probe_grid() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

// 8-value groups the fragments are drawn from (bounded for 32-bit indexing)
uint32_t groups_of(int64_t elems) {
  const int64_t g = elems / 8;
  return (uint32_t)(g > (int64_t(1) << 30) ? (int64_t(1) << 30) : (g < 1 ? 1 : g));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace lmh

LMH_API size_t lmhead_mfma_probe_workspace_bytes(void) {
  const size_t g = (size_t)lmh::probe_grid();
  return g * sizeof(unsigned long long) + g * lmh::kThreads * sizeof(float);
}

LMH_API int lmhead_mfma_probe(const void* a, int64_t a_elems, const void* b, int64_t b_elems,
                              int64_t iters, void* workspace, size_t workspace_bytes,
                              double* ms, double* flops, double* clock_ghz, void* stream) {
  using namespace lmh;
  if (iters <= 0 || iters > kProbeMaxIters) return LMHEAD_ERR_INVALID_ARG;
  if ((a == nullptr) != (b == nullptr)) return LMHEAD_ERR_INVALID_ARG;
  if (a != nullptr && (a_elems < 8 || b_elems < 8 || !aligned16(a) || !aligned16(b)))
    return LMHEAD_ERR_INVALID_ARG;
  if (workspace == nullptr || !aligned16(workspace)) return LMHEAD_ERR_INVALID_ARG;
  const int grid = probe_grid();
  if (workspace_bytes < lmhead_mfma_probe_workspace_bytes()) return LMHEAD_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto* cycles = reinterpret_cast<unsigned long long*>(workspace);
  float* sink = reinterpret_cast<float*>(cycles + grid);

  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return LMHEAD_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return LMHEAD_ERR_HIP;
  }
  int st = LMHEAD_OK;
  float elapsed = 0.f;
  std::vector<unsigned long long> host(grid);
  if (hipEventRecord(e0, s) != hipSuccess) st = LMHEAD_ERR_HIP;
  if (st == LMHEAD_OK) {
    if (lmh_launch::launch_kernel(k_mfma_probe, dim3(grid), dim3(kThreads), s,
                                  reinterpret_cast<const uint16_t*>(a), groups_of(a_elems),
                                  reinterpret_cast<const uint16_t*>(b), groups_of(b_elems),
                                  (int)iters, cycles, sink) != hipSuccess)
      st = LMHEAD_ERR_HIP;
  }
  if (st == LMHEAD_OK && hipEventRecord(e1, s) != hipSuccess) st = LMHEAD_ERR_HIP;
  if (st == LMHEAD_OK && hipEventSynchronize(e1) != hipSuccess) st = LMHEAD_ERR_HIP;
  if (st == LMHEAD_OK && hipEventElapsedTime(&elapsed, e0, e1) != hipSuccess) st = LMHEAD_ERR_HIP;
  if (st == LMHEAD_OK &&
      hipMemcpyAsync(host.data(), cycles, grid * sizeof(unsigned long long),
                     hipMemcpyDeviceToHost, s) != hipSuccess)
    st = LMHEAD_ERR_HIP;
  if (st == LMHEAD_OK && hipStreamSynchronize(s) != hipSuccess) st = LMHEAD_ERR_HIP;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != LMHEAD_OK) return st;

  // 64 MFMAs of 2 * 16 * 16 * 32 flops per set and iteration, per wave
  const double fl = (double)grid * kProbeWavesPerGroup * (double)iters * kProbeSets * 64.0 *
                    (2.0 * 16 * 16 * 32);
  double cyc = 0.0;
  for (int i = 0; i < grid; ++i) cyc += (double)host[i];
  cyc /= grid;
  if (ms) *ms = elapsed;
  if (flops) *flops = fl;
  if (clock_ghz) *clock_ghz = elapsed > 0.f ? cyc / (elapsed * 1e-3) / 1e9 : 0.0;
  return LMHEAD_OK;
}
