// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A[m][k] * B[n][k] with v_mfma_f32_32x32x16_bf16.
// Both operands are K-major (row-major with k contiguous): every GEMM of the
// op is arranged that way, using transposed copies where needed. Each wave
// owns a 128 x 128 sub-tile held as 4 x 4 MFMA accumulator blocks (256 AGPRs).
//
// K advances in stages of 32 through a ring of 4 LDS stages. Stages are loaded
// straight from global memory into LDS with buffer_load_dwordx4 ... lds (no
// VGPR staging); the buffer descriptor's record count zero-fills rows past
// the end of the matrix. Loads run 4 stages ahead; one barrier per stage both
// publishes stage k+1 and frees the buffer of stage k for stage k+4. MFMA
// fragments are double-buffered in registers: the fragments of the next
// 16-wide k step are read from LDS while the current step's 16 MFMAs issue.
//
// LDS stage layout: a tile row (an m of A or an n of B) holds its 32 k values
// as four 16-byte chunks; the chunk index is XOR-swizzled with (row >> 2) & 3.
// With that swizzle the MFMA fragment reads (lane l reads row l % 32, chunk
// 2 kk + l / 32) showed zero LDS bank-conflict cycles on gfx950 in a counter
// measurement of ds_read_b128 address patterns, and each direct-to-LDS load
// still writes 1 KiB contiguously.
//
// MFMA 32x32x16 bf16 register layout (lane l of 64):
//   A fragment: row  l % 32, k = 8 * (l / 32) + [0..7]
//   B fragment: col  l % 32, k = 8 * (l / 32) + [0..7]
//   D (16 fp32): col l % 32, row = 8 * (r / 4) + 4 * (l / 32) + (r % 4)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 32;
constexpr int kStages = 4;
constexpr int kThreads = 256;
constexpr int kOperandStageBytes = kBM * kBK * 2;            // 16 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;          // A then B
constexpr int kRingBytes = kStages * kStageBytes;            // 128 KiB
constexpr int kLdsBytes = kRingBytes;
constexpr int kLoadsPerWaveStage = 2 * (kOperandStageBytes / 4 / 1024);  // 8
constexpr uint32_t kOOB = 0x80000000u;  // voffset beyond every record count
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ int lds_swz(int row) { return (row >> 2) & 3; }

// Byte offset of (row, 16-byte chunk) inside one operand stage.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row * 4 + (chunk ^ lds_swz(row))) * 16;
}

// s_waitcnt with the given vmcnt and no wait on the other counters (gfx9
// encoding: vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14).
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// A K-major operand tile source: rows row0 .. row0 + 255 of a [rows][ld]
// bf16 matrix; rows at or past `rows_valid` read as zero.
struct TileSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[4];  // per load instruction: byte offset of this lane's chunk at k = 0

  // tile_base: element pointer of the tile's first row; ld: row pitch
  // (elements, multiple of 8); rows: rows of this tile inside the matrix.
  __device__ __forceinline__ void init(const uint16_t* tile_base, int64_t ld, int rows) {
    rows = rows < 0 ? 0 : (rows > kBM ? kBM : rows);
    // The descriptor must live in SGPRs: pass its inputs through readfirstlane
    // so the compiler sees them as wave-uniform (they are uniform by design).
    const uint64_t p = reinterpret_cast<uint64_t>(tile_base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const int bytes = __builtin_amdgcn_readfirstlane((int)((int64_t)rows * ld * 2));
    void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kRsrcWord3);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wave * 64 + j * 16 + (lane >> 2);
      const int c = (lane & 3) ^ lds_swz(row);
      off[j] = row < rows ? (uint32_t)(row * ld * 2 + c * 16) : kOOB;
    }
  }
  // Issue this wave's 4 loads of stage kt into the operand stage at `dst`.
  __device__ __forceinline__ void issue(int kt, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* base = dst + wave * 4096;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(base + j * 1024), 16,
                                               off[j] + (uint32_t)(kt * kBK * 2), 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Tile scheduling: persistent workgroups, XCD-aware grouped order.
// Workgroups are dispatched round-robin over the 8 XCDs (chiplets), so block
// b runs on XCD b % 8. Slot b of round `r` is remapped so that the blocks of
// one XCD take consecutive logical tiles; logical tiles run in groups of
// kGroupM m-tiles by all n-tiles (m fastest inside a group), so the 32
// concurrent tiles of an XCD form a 4 x 8 block sharing A and B panels in
// that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ int xcd_logical(int round, int grid) {
  const int b = blockIdx.x;
  const int per = grid / kXcds;  // grid is a multiple of kXcds
  return round * grid + (b % kXcds) * per + (b / kXcds);
}

__device__ __forceinline__ void tile_coords(int t, int mt, int nt, int& tm, int& tn) {
  const int per_group = kGroupM * nt;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = min(mt - first, kGroupM);
  const int r = t - g * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

// ---------------------------------------------------------------------------
// Main loop.
// ---------------------------------------------------------------------------
struct Frags {
  bf16x8_t a[4], b[4];
};

__device__ __forceinline__ void read_frags(const char* stage, int kk, int lane, int wm, int wn,
                                           Frags& f) {
  const int r = lane & 31;
  const int c = kk * 2 + (lane >> 5);
  const int o = lds_off(r, c);  // swizzle depends only on lane & 31 (see header)
  const char* a = stage + wm * 128 * 64 + o;
  const char* b = stage + kOperandStageBytes + wn * 128 * 64 + o;
  // first-use order of mfma_step: a0 with b0..b3, then a1, a2, a3
  f.a[0] = *reinterpret_cast<const bf16x8_t*>(a);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const bf16x8_t*>(b + j * 32 * 64);
#pragma unroll
  for (int i = 1; i < 4; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(a + i * 32 * 64);
}

__device__ __forceinline__ void mfma_step(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void issue_stage(const TileSrc& A, const TileSrc& B, int kt,
                                            char* ring) {
  char* st = ring + (kt % kStages) * kStageBytes;
  A.issue(kt, st);
  B.issue(kt, st + kOperandStageBytes);
}

// Waits until at most `ahead` stages of this wave's loads are in flight.
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
  if (ahead >= 3)
    wait_vmcnt<3 * kLoadsPerWaveStage>();
  else if (ahead == 2)
    wait_vmcnt<2 * kLoadsPerWaveStage>();
  else if (ahead == 1)
    wait_vmcnt<kLoadsPerWaveStage>();
  else
    wait_vmcnt<0>();
}

// One k step of kBK: the fragments of kk = 0 (f0) are in registers; read
// kk = 1 (f1), run f0's MFMAs, publish stage kt + 1 (wait + barrier), start the
// loads of stage kt + kStages into the buffer stage kt used, read the next
// stage's kk = 0 fragments, run f1's MFMAs. STEADY: every condition is known
// true (kt + kStages < nk), so the body is straight-line code.
// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

template <bool STEADY>
__device__ __forceinline__ void k_step(const TileSrc& A, const TileSrc& B, int kt, int nk,
                                       char* ring, int lane, int wm, int wn, Frags& f0, Frags& f1,
                                       f32x16_t (&acc)[4][4]) {
  const char* st = ring + (kt % kStages) * kStageBytes;
  // sched_barrier(0) fences keep the phases in this order: the compiler would
  // otherwise interleave them to shorten live ranges, which serialises LDS
  // latency against the MFMAs.
  read_frags(st, 1, lane, wm, wn, f1);
  mfma_step(f0, acc);
  // one LDS read between consecutive MFMAs, so MFMA issue never waits on them
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (STEADY) {
    wait_vmcnt<2 * kLoadsPerWaveStage>();  // stage kt + 1 landed (kt + 2, kt + 3 may fly)
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_stage(A, B, kt + kStages, ring);
    read_frags(ring + ((kt + 1) % kStages) * kStageBytes, 0, lane, wm, wn, f0);
    mfma_step(f1, acc);
    // loads and next-stage fragment reads threaded between f1's MFMAs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 1);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    return;
  } else if (kt + 1 < nk) {
    // stages issued so far: 0 .. min(nk - 1, kt + kStages - 1)
    const int last = (nk - 1 < kt + kStages - 1) ? nk - 1 : kt + kStages - 1;
    wait_stages_ahead(last - (kt + 1));
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (kt + kStages < nk) issue_stage(A, B, kt + kStages, ring);
    read_frags(ring + ((kt + 1) % kStages) * kStageBytes, 0, lane, wm, wn, f0);
  } else {
    wait_lgkm0();
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(f1, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// Accumulates the tile over nk stages of kBK. The caller must have made the
// LDS ring free (barrier) before the call; on return every wave has finished
// its LDS reads and no load is in flight.
__device__ __forceinline__ void mainloop(const TileSrc& A, const TileSrc& B, int nk, char* ring,
                                         f32x16_t (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;

  const int pro = nk < kStages ? nk : kStages;
  for (int s = 0; s < pro; ++s) issue_stage(A, B, s, ring);
  wait_stages_ahead(pro - 1);
  __builtin_amdgcn_s_barrier();

  Frags f0, f1;
  read_frags(ring, 0, lane, wm, wn, f0);
  int kt = 0;
  for (; kt + kStages < nk; ++kt) k_step<true>(A, B, kt, nk, ring, lane, wm, wn, f0, f1, acc);
  for (; kt < nk; ++kt) k_step<false>(A, B, kt, nk, ring, lane, wm, wn, f0, f1, acc);
  wait_lgkm0();
}

// Row (within the wave's 128-row half) held by accumulator register r of block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace lmh
