// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A[m][k] * B[n][k] with v_mfma_f32_32x32x16_bf16.
// Both operands are K-major (row-major with k contiguous): every GEMM of the
// op is arranged that way, using transposed copies where needed. Each wave
// owns a 128 x 128 sub-tile held as 4 x 4 MFMA accumulator blocks (256 AGPRs).
//
// K advances in stages of 32 through a ring of 5 LDS stages (160 KiB). Stages are loaded
// straight from global memory into LDS with buffer_load_dwordx4 ... lds (no
// VGPR staging); the buffer descriptor's record count zero-fills rows past
// the end of the matrix. Loads run kStages stages ahead; one barrier per stage both
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
constexpr int kBK = 64;                                      // k per stage
constexpr int kChunks = kBK / 8;                             // 16-byte chunks per row
constexpr int kRowBytes = kBK * 2;                           // 128: one L2 line per row
constexpr int kStages = 2;
constexpr int kThreads = 256;
constexpr int kOperandStageBytes = kBM * kRowBytes;          // 32 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;          // A then B
constexpr int kRingBytes = kStages * kStageBytes;            // 128 KiB
constexpr int kRowsPerLoad = 1024 / kRowBytes;               // rows per 1 KiB LDS-DMA load
constexpr int kLoadsPerWaveOperand = (kBM / 4) / kRowsPerLoad;  // 8
constexpr int kLoadsPerWaveStage = 2 * kLoadsPerWaveOperand;    // 16
constexpr uint32_t kOOB = 0x80000000u;  // voffset beyond every record count
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & (kChunks - 1); }

// Byte offset of (row, 16-byte chunk) inside one operand stage.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row * kChunks + (chunk ^ lds_swz(row))) * 16;
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
  __amdgpu_buffer_rsrc_t none;          // zero records: every load reads zeros
  uint32_t off[kLoadsPerWaveOperand];  // per load: byte offset of this lane's chunk at k = 0

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
    none = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0, kRsrcWord3);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kLoadsPerWaveOperand; ++j) {
      const int row = wave * (kBM / 4) + j * kRowsPerLoad + lane / kChunks;
      const int c = (lane % kChunks) ^ lds_swz(row);
      off[j] = row < rows ? (uint32_t)(row * ld * 2 + c * 16) : kOOB;
    }
  }
  // Issue this wave's loads of stage kt into the operand stage at `dst`;
  // stages at or past nk read as zeros (zero-record descriptor).
  __device__ __forceinline__ void issue(int kt, int nk, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* base = dst + wave * (kBM / 4) * kRowBytes;
    // the k offset rides in the scalar soffset field; rows past the end keep
    // voffset >= the record count whether or not soffset enters the check
    const bool live = kt < nk;
    const int koff = __builtin_amdgcn_readfirstlane(live ? kt * kRowBytes : 0);
    const __amdgpu_buffer_rsrc_t r = live ? rsrc : none;
#pragma unroll
    for (int j = 0; j < kLoadsPerWaveOperand; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + j * 1024), 16, off[j], koff,
                                               0, 0);
  }
};

// ---------------------------------------------------------------------------
// Tile scheduling: persistent workgroups, XCD-aware grouped order.
// Workgroups are dispatched round-robin over the 8 XCDs (chiplets), so block
// b runs on XCD b % 8. Slot b of round `r` is remapped so that the blocks of
// one XCD take consecutive logical tiles; logical tiles run in groups of
// GM m-tiles by all n-tiles (m fastest inside a group), so the 32
// concurrent tiles of an XCD form a GM x (32 / GM) block sharing A and B
// panels in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
// Group widths (m-tiles per group) of each GEMM, chosen by a timing sweep
// over 1..32 at N=16384 H=4096 V=131072; a group is swept with m
// fastest, so an XCD's 32 concurrent tiles cover gm m-tiles by 32 / gm n-tiles.
#ifndef LMH_GM_FWD
#define LMH_GM_FWD 8
#endif
#ifndef LMH_GM_DZ
#define LMH_GM_DZ 8
#endif
#ifndef LMH_GM_DX
#define LMH_GM_DX 16
#endif
#ifndef LMH_GM_DW
#define LMH_GM_DW 16
#endif

__device__ __forceinline__ int xcd_logical(int round, int grid) {
  const int b = blockIdx.x;
  const int per = grid / kXcds;  // grid is a multiple of kXcds
  return round * grid + (b % kXcds) * per + (b / kXcds);
}

template <int GM>
__device__ __forceinline__ void tile_coords(int t, int mt, int nt, int& tm, int& tn) {
  const int per_group = GM * nt;
  const int g = t / per_group;
  const int first = g * GM;
  const int gm = min(mt - first, GM);
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
  const char* a = stage + wm * 128 * kRowBytes + o;
  const char* b = stage + kOperandStageBytes + wn * 128 * kRowBytes + o;
  // first-use order of mfma_step: a0 with b0..b3, then a1, a2, a3
  f.a[0] = *reinterpret_cast<const bf16x8_t*>(a);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const bf16x8_t*>(b + j * 32 * kRowBytes);
#pragma unroll
  for (int i = 1; i < 4; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(a + i * 32 * kRowBytes);
}

__device__ __forceinline__ void mfma_step(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void issue_stage(const TileSrc& A, const TileSrc& B, int kt, int nk,
                                            char* st) {
  A.issue(kt, nk, st);
  B.issue(kt, nk, st + kOperandStageBytes);
}

// Waits until at most `ahead` stages of this wave's loads are in flight.
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
  static_assert(kStages <= 3, "extend the cases below");
  if (ahead >= 2)
    wait_vmcnt<2 * kLoadsPerWaveStage>();
  else if (ahead == 1)
    wait_vmcnt<kLoadsPerWaveStage>();
  else
    wait_vmcnt<0>();
}

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// Runs one 16-wide MFMA k step from `cur` while reading the fragments of k
// step `kk` of `stage` into `nxt`, one LDS read between consecutive MFMAs.
template <int ID>
__device__ __forceinline__ void step_and_read(const char* stage, int kk, int lane, int wm, int wn,
                                              const Frags& cur, Frags& nxt,
                                              f32x16_t (&acc)[4][4]) {
  read_frags(stage, kk, lane, wm, wn, nxt);
  mfma_step(cur, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, ID);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, ID);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, ID);
  __builtin_amdgcn_sched_barrier(0);
}

// The two LDS ring slots are separate __shared__ objects (slot0, slot1) and
// the loop is unrolled by two, so every LDS access names a fixed slot: the
// compiler can then see that a stage's fragment reads never alias the
// direct-to-LDS loads in flight into the other slot, and inserts no waits.
struct Ring {
  char* slot[kStages];
};

// One stage of kBK = 4 MFMA k steps from slot `cur`. On entry f0 holds the
// stage's kk = 0 fragments. kk = 1..3 are read from LDS while the previous k
// step's MFMAs issue; before the last k step every wave publishes stage kt + 1
// (wait + barrier), the loads of stage kt + 2 go into `cur`, and the next
// stage's kk = 0 fragments are read from `nxt` during the last 16 MFMAs.
// Every stage runs this same straight-line body: stages past the end of K are
// zeros, so the loop can run in pairs over an even number of stages.
__device__ __forceinline__ void k_step(const TileSrc& A, const TileSrc& B, int kt, int nk,
                                       char* cur, char* nxt, int lane, int wm, int wn, Frags& f0,
                                       Frags& f1, f32x16_t (&acc)[4][4]) {
  __builtin_amdgcn_sched_barrier(0);
  step_and_read<0>(cur, 1, lane, wm, wn, f0, f1, acc);
  step_and_read<1>(cur, 2, lane, wm, wn, f1, f0, acc);
  step_and_read<2>(cur, 3, lane, wm, wn, f0, f1, acc);
  // stage kt + 1 must have landed; with two stages nothing newer is in flight
  wait_vmcnt<0>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  issue_stage(A, B, kt + kStages, nk, cur);
  read_frags(nxt, 0, lane, wm, wn, f0);
  mfma_step(f1, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 3);
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 3);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 3);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 3);
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 3);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Accumulates the tile over nk stages of kBK. The caller must have made the
// LDS ring free (barrier) before the call; on return every wave has finished
// its LDS reads and no load is in flight.
__device__ __forceinline__ void mainloop(const TileSrc& A, const TileSrc& B, int nk, char* slot0,
                                         char* slot1, f32x16_t (&acc)[4][4]) {
  static_assert(kStages == 2, "the loop below is unrolled for a two-slot ring");
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

  issue_stage(A, B, 0, nk, slot0);
  issue_stage(A, B, 1, nk, slot1);
  wait_vmcnt<kLoadsPerWaveStage>();
  __builtin_amdgcn_s_barrier();

  Frags f0, f1;
  read_frags(slot0, 0, lane, wm, wn, f0);
  for (int kt = 0; kt < nk; kt += 2) {
    k_step(A, B, kt, nk, slot0, slot1, lane, wm, wn, f0, f1, acc);
    k_step(A, B, kt + 1, nk, slot1, slot0, lane, wm, wn, f0, f1, acc);
  }
  // the last pair issued two zero stages that nobody reads; let them land
  wait_vmcnt<0>();
  wait_lgkm0();
}

// Row (within the wave's 128-row half) held by accumulator register r of block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace lmh
