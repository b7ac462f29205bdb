// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A[m][k] * B[n][k] with v_mfma_f32_32x32x16_bf16.
// Each wave owns a 128 x 128 sub-tile held as 4 x 4 MFMA accumulator blocks
// (256 AGPRs).
//
// An operand is read from global memory in one of two layouts, chosen per GEMM
// so that no operand ever needs a transposed copy:
//   KSrc  : K-major, [mn][ld] with k contiguous (e.g. W[v][h] as the A of
//           Z = W X^T, K = h);
//   MNSrc : MN-major, [k][ld] with mn contiguous (e.g. W[v][h] as the B of
//           dX = dZ W, K = v, n = h).
//
// K advances in stages of kBK = 32 through a ring of four LDS stages (4 x
// 32 KiB). Stages are loaded straight from global memory into LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging); the buffer descriptor's
// record count zero-fills rows past the end of the matrix. The loads of stage
// k + 3 go into the slot that stage k - 1 released and are spread over the
// whole of stage k, one load per four MFMAs: a CU moves about 150 GB/s through
// these loads, twice what the MFMAs consume on average, so loads bunched into
// a fraction of a stage would stall the issuing wave. One barrier per stage
// publishes stage k + 1 and releases the slot of stage k. MFMA fragments are
// double-buffered in registers: the fragments of the next 16-wide k step are
// read from LDS while the current step's 16 MFMAs issue.
//
// LDS stage layouts (16 KiB per operand, 256 mn x 32 k bf16):
//   K-major : 256 rows (one per m or n) of 64 bytes (32 k); the 16-byte chunk
//             index is XOR-swizzled with (row >> 2) & 3, which keeps the
//             fragment reads (ds_read_b128, lane l: row l % 32, chunk
//             2 kk + l / 32) free of bank conflicts.
//   MN-major: 8 groups of 4 consecutive k rows, 2 KiB each. Inside a group
//             the 64-byte piece (32 mn values) of k row e in 32-wide mn block
//             s sits at byte (4 s + e) * 64, i.e. the four k rows are
//             interleaved piece by piece. Fragments are read with
//             ds_read_b64_tr_b16, which hands lane i of each 16-lane group
//             element i % 4 of the 8 bytes addressed by lane 4 e + i / 4 as its
//             element e: pointing lane 4 e + q at k row k0 + e, mn n0 + 4 q
//             gives lane i the values (mn n0 + i, k k0 .. k0 + 3), which is the
//             MFMA fragment shape; two such reads give the 8 k of a fragment.
//             A half wave reads 4 whole pieces that are adjacent in LDS
//             (256 contiguous bytes), so the reads are free of bank conflicts,
//             and one direct-to-LDS load (1 KiB) fills half a group from
//             4 rows x 256 contiguous global bytes.
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
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 32;                                      // k per stage
constexpr int kChunks = kBK / 8;                             // 16-byte chunks per K-major row
constexpr int kRowBytes = kBK * 2;                           // 64: half an L2 line per row
constexpr int kStages = 4;
constexpr int kThreads = 256;
constexpr int kOperandStageBytes = kBM * kRowBytes;          // 16 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;          // A then B
constexpr int kRingBytes = kStages * kStageBytes;            // 128 KiB
constexpr int kRowsPerLoad = 1024 / kRowBytes;               // rows per 1 KiB LDS-DMA load
constexpr int kLoadsPerWaveOperand = (kBM / 4) / kRowsPerLoad;  // 4
constexpr int kLoadsPerWaveStage = 2 * kLoadsPerWaveOperand;    // 8
constexpr uint32_t kOOB = 0x80000000u;  // voffset beyond every record count
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// MN-major stage geometry
constexpr int kMnRowBytes = kBM * 2;                // 512: one k row of 256 mn values
constexpr int kMnGroupBytes = 4 * kMnRowBytes;      // 2 KiB: 4 interleaved k rows
constexpr int kMnPieceBytes = 64;                   // 32 mn values of one k row
static_assert(kBK / 4 * kMnGroupBytes == kOperandStageBytes, "MN-major stage size");

__device__ __forceinline__ int lds_swz(int row) { return (row >> 2) & (kChunks - 1); }

// Byte offset of (row, 16-byte chunk) inside one K-major operand stage.
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

// A buffer descriptor must live in SGPRs: its inputs go through readfirstlane
// so the compiler sees them as wave-uniform (they are uniform by design).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// A K-major operand tile source: rows row0 .. row0 + 255 of a [rows][ld]
// bf16 matrix; rows at or past `rows_valid` read as zero.
struct KSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  __amdgpu_buffer_rsrc_t none;          // zero records: every load reads zeros
  uint32_t off[kLoadsPerWaveOperand];  // per load: byte offset of this lane's chunk at k = 0

  // tile_base: element pointer of the tile's first row; ld: row pitch
  // (elements, multiple of 8); rows: rows of this tile inside the matrix.
  __device__ __forceinline__ void init(const uint16_t* tile_base, int64_t ld, int rows) {
    rows = rows < 0 ? 0 : (rows > kBM ? kBM : rows);
    const int bytes = __builtin_amdgcn_readfirstlane((int)((int64_t)rows * ld * 2));
    void* base = reinterpret_cast<void*>(uniform_u64(reinterpret_cast<uint64_t>(tile_base)));
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
  // Fragment of k step kk, 32-row block i of the wave's 128-row half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* op, int kk, int lane, int half,
                                                  int i) {
    const int o = lds_off(lane & 31, kk * 2 + (lane >> 5));  // swizzle depends on lane & 31 only
    return *reinterpret_cast<const bf16x8_t*>(op + (half * 128 + i * 32) * kRowBytes + o);
  }
  static constexpr int kReadsPerFrag = 1;
};

// An MN-major operand tile source: columns mn0 .. mn0 + 255 of the k rows of a
// [k_rows][ld] bf16 matrix (mn contiguous); k rows at or past k_rows and
// columns at or past mn_valid (counted from mn0) read as zero.
struct MNSrc {
  uint64_t base;                        // byte address of (k 0, mn0); wave-uniform
  int64_t pitch;                        // bytes per k row; wave-uniform
  int k_valid;                          // wave-uniform
  uint32_t off[kLoadsPerWaveOperand];  // per load: byte offset of this lane's chunk in a stage

  __device__ __forceinline__ void init(const uint16_t* col_base, int64_t ld, int k_rows,
                                       int mn_valid) {
    base = uniform_u64(reinterpret_cast<uint64_t>(col_base));
    pitch = (int64_t)uniform_u64((uint64_t)(ld * 2));
    k_valid = __builtin_amdgcn_readfirstlane(k_rows < 0 ? 0 : k_rows);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = (lane >> 2) & 3;     // k row inside the group
    const int blk = lane >> 4;         // 32-wide mn block inside the half
    const int cq = lane & 3;           // 16-byte chunk inside the piece
#pragma unroll
    for (int j = 0; j < kLoadsPerWaveOperand; ++j) {
      // load j fills half (j & 1) of group kGroupsPerWave wave + j / 2 of the stage
      const int row = (wave * kGroupsPerWave + (j >> 1)) * 4 + e;
      const int col = ((j & 1) * 4 + blk) * 32 + cq * 8;
      off[j] = col < mn_valid ? (uint32_t)(row * pitch + col * 2) : kOOB;
    }
  }
  // Issue this wave's loads of stage kt into the operand stage at `dst`. The
  // descriptor is rebased to the stage's first k row, and its record count
  // covers only the valid rows of the stage (none at or past k_valid).
  __device__ __forceinline__ void issue(int kt, int /*nk*/, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* ldsb = dst + wave * kGroupsPerWave * kMnGroupBytes;
    int rows = k_valid - kt * kBK;
    rows = rows < 0 ? 0 : (rows > kBK ? kBK : rows);
    void* p = reinterpret_cast<void*>(uniform_u64(base + (uint64_t)((int64_t)kt * kBK * pitch)));
    const int bytes = __builtin_amdgcn_readfirstlane((int)(rows * pitch));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes,
                                                                       kRsrcWord3);
#pragma unroll
    for (int j = 0; j < kLoadsPerWaveOperand; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(ldsb + (j >> 1) * kMnGroupBytes + (j & 1) * 1024), 16, off[j], 0, 0, 0);
  }
  static __device__ __forceinline__ bf16x4_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(lds_ptr_t)(p));
  }
  // Fragment of k step kk, 32-wide mn block i of the wave's 128 half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* op, int kk, int lane, int half,
                                                  int i) {
    // lane 16 g + 4 e + q reads k row 16 kk + 8 (g >> 1) + 4 h + e at mn
    // 128 half + 32 i + 16 (g & 1) + 4 q, for the two halves h of the fragment
    const int g = lane >> 4;
    const int lane_part = (g >> 1) * 2 * kMnGroupBytes + ((lane >> 2) & 3) * kMnPieceBytes +
                          (g & 1) * 32 + (lane & 3) * 8;
    const char* p = op + kk * 4 * kMnGroupBytes + (half * 4 + i) * 4 * kMnPieceBytes + lane_part;
    const bf16x4_t lo = tr_read(p);
    const bf16x4_t hi = tr_read(p + kMnGroupBytes);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static constexpr int kReadsPerFrag = 2;
  static constexpr int kGroupsPerWave = kBK / 4 / 4;  // 4-row groups each wave loads per stage
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
// Group widths (m-tiles per group) of each GEMM; a group is swept with m
// fastest, so an XCD's 32 concurrent tiles cover gm m-tiles by 32 / gm n-tiles
// and read gm + 32 / gm operand panels (12 for gm = 8, the fewest). Timed at
// N=16384 H=4096 V=131072 on random operands, 4 and 8 tie and 16 is slower.
#ifndef LMH_GM_FWD
#define LMH_GM_FWD 8
#endif
#ifndef LMH_GM_DZ
#define LMH_GM_DZ 8
#endif
#ifndef LMH_GM_DX
#define LMH_GM_DX 8
#endif
#ifndef LMH_GM_DW
#define LMH_GM_DW 8
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
// The ring's slots must be distinct __shared__ objects named at every access
// (see mainloop); kernels declare them with this macro.
#define LMH_DECLARE_RING                                                  \
  __shared__ __attribute__((aligned(1024))) char slot0[lmh::kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char slot1[lmh::kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char slot2[lmh::kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char slot3[lmh::kStageBytes]
struct Frags {
  bf16x8_t a[4], b[4];
};

template <class SA, class SB>
__device__ __forceinline__ void read_frags(const char* stage, int kk, int lane, int wm, int wn,
                                           Frags& f) {
  const char* a = stage;
  const char* b = stage + kOperandStageBytes;
  // first-use order of mfma_step: a0 with b0..b3, then a1, a2, a3
  f.a[0] = SA::frag(a, kk, lane, wm, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = SB::frag(b, kk, lane, wn, j);
#pragma unroll
  for (int i = 1; i < 4; ++i) f.a[i] = SA::frag(a, kk, lane, wm, i);
}

__device__ __forceinline__ void mfma_step(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// LDS read instructions per 16-wide k step for operand layouts SA, SB (8..16).
template <class SA, class SB>
constexpr int reads_per_step() {
  return 4 * (SA::kReadsPerFrag + SB::kReadsPerFrag);
}

// Interleaves the 16 MFMAs of a k step with its LDS reads (one after each
// MFMA) and, with LOADS, the kLoadsPerWaveOperand loads of one operand (one
// per four MFMAs).
template <class SA, class SB, bool LOADS, int ID>
__device__ __forceinline__ void interleave() {
  constexpr int nr = reads_per_step<SA, SB>();
  constexpr int every = 16 / kLoadsPerWaveOperand;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, ID);
    if (LOADS && i % every == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, ID);
    if (i < nr) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, ID);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One stage of kBK = 2 MFMA k steps from slot `cur`. On entry f0 holds the
// stage's kk = 0 fragments and slot `fre` is free (its stage kt - 1 was
// released by the previous barrier). Step 1 runs kk = 0 while reading kk = 1
// into f1 and issuing stage kt + 3's A loads into `fre`. Then every wave
// waits for its loads of stage kt + 1 (at most the 8 loads of stage kt + 2
// and the 4 just issued may remain) and for its LDS reads, and the barrier
// publishes stage kt + 1 and releases `cur`. Step 2 runs kk = 1 while reading
// stage kt + 1's kk = 0 fragments from `nxt` and issuing stage kt + 3's B loads.
// Stages past the end of K are zeros, so every stage runs this same body.
template <class SA, class SB>
__device__ __forceinline__ void k_stage(const SA& A, const SB& B, int kt, int nk, const char* cur,
                                        const char* nxt, char* fre, int lane, int wm, int wn,
                                        Frags& f0, Frags& f1, f32x16_t (&acc)[4][4]) {
  static_assert(kStages == 4 && kLoadsPerWaveOperand == 4, "waits below assume this ring");
  __builtin_amdgcn_sched_barrier(0);
  read_frags<SA, SB>(cur, 1, lane, wm, wn, f1);
  A.issue(kt + 3, nk, fre);
  mfma_step(f0, acc);
  interleave<SA, SB, true, 0>();
  wait_vmcnt<kLoadsPerWaveStage + kLoadsPerWaveOperand>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags<SA, SB>(nxt, 0, lane, wm, wn, f0);
  B.issue(kt + 3, nk, fre + kOperandStageBytes);
  mfma_step(f1, acc);
  interleave<SA, SB, true, 1>();
}

// Accumulates the tile over nk stages of kBK. The caller must have made the
// LDS ring free (barrier) before the call; on return every wave has finished
// its LDS reads and no load is in flight. The four slots are distinct
// __shared__ objects and the loop is unrolled by four, so every LDS access
// names a fixed slot: the compiler can then see that fragment reads never
// alias the direct-to-LDS loads in flight into other slots, and inserts no
// waits of its own.
template <class SA, class SB>
__device__ __forceinline__ void mainloop(const SA& A, const SB& B, int nk, char* slot0,
                                         char* slot1, char* slot2, char* slot3,
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

  A.issue(0, nk, slot0);
  B.issue(0, nk, slot0 + kOperandStageBytes);
  A.issue(1, nk, slot1);
  B.issue(1, nk, slot1 + kOperandStageBytes);
  A.issue(2, nk, slot2);
  B.issue(2, nk, slot2 + kOperandStageBytes);
  wait_vmcnt<2 * kLoadsPerWaveStage>();
  __builtin_amdgcn_s_barrier();

  Frags f0, f1;
  read_frags<SA, SB>(slot0, 0, lane, wm, wn, f0);
  for (int kt = 0; kt < nk; kt += 4) {
    k_stage(A, B, kt, nk, slot0, slot1, slot3, lane, wm, wn, f0, f1, acc);
    k_stage(A, B, kt + 1, nk, slot1, slot2, slot0, lane, wm, wn, f0, f1, acc);
    k_stage(A, B, kt + 2, nk, slot2, slot3, slot1, lane, wm, wn, f0, f1, acc);
    k_stage(A, B, kt + 3, nk, slot3, slot0, slot2, lane, wm, wn, f0, f1, acc);
  }
  // the last stages issued zero loads that nobody reads; let them land
  wait_vmcnt<0>();
  wait_lgkm0();
}

// Row (within the wave's 128-row half) held by accumulator register r of
// block i: acc_row_fixed(i, r) + acc_row_lane(lane). Epilogues compare the
// compile-time part against a per-tile lane bound, so the compiler has no
// per-register lane values to keep live across the tile loop.
__host__ __device__ constexpr int acc_row_fixed(int i, int r) {
  return i * 32 + 8 * (r >> 2) + (r & 3);
}
__device__ __forceinline__ int acc_row_lane(int lane) { return 4 * (lane >> 5); }

}  // namespace lmh
