// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A[m][k] * B[n][k] with v_mfma_f32_16x16x32_bf16.
// Each wave owns a 128 x 128 sub-tile held as 8 x 8 MFMA accumulator blocks
// of 16 x 16 (256 AGPRs).
//
// Why 16 x 16 x 32: under this load the chip runs at the clock its power
// limit allows, and at equal flops the 16 x 16 x 32 instruction draws less
// power than 32 x 32 x 16 (it moves half the accumulator bytes per flop).
// With operands in registers and the bench batch's bit statistics, measured
// on MI355X: 16 x 16 x 32 reaches 2.05 PFLOP/s at 2.00 GHz, 32 x 32 x 16
// 1.81 PFLOP/s at 1.73 GHz. Per k step of 32 the two shapes read the same
// operand bytes from LDS.
//
// Operand layouts in global memory, one of each per GEMM:
//   A : K-major, [m][ld] with k contiguous (e.g. W[v][h] for Z = W X^T);
//   B : MN-major, [k][ld] with n contiguous (e.g. W[v][h] for dX = dZ W).
// Every GEMM of the op can be arranged this way without a transposed copy of
// a large operand.
//
// Both operands are loaded straight from global memory into LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging); a buffer descriptor's record
// count zero-fills rows past the end of a matrix. K advances in stages of
// kBK = 32, one MFMA k step of 64 MFMAs per wave; each stage issues four
// loads per wave for each operand, spread over the stage's MFMAs. MFMA
// fragments are double-buffered in registers: while a stage's 64 MFMAs
// issue, the fragments of the next stage are read from LDS, spread over the
// stage. One barrier per stage, at its start, publishes the next stage (whose
// fragments the stage reads) and releases the LDS of the current one (whose
// fragments were read during the previous stage).
//
// LDS (160 KiB, all of it):
//   A ring: three slots of one k pair (64 k, two stages), 32 KiB each. A row
//     of the pair is 128 bytes, one whole L2 line: fetching K-major rows 64
//     bytes at a time would split every line across two requests, and the L2
//     fetches each 64-byte sector on its own miss. The 16-byte chunk index
//     is XOR-swizzled with (row >> 1) & 7, which keeps the fragment reads
//     (ds_read_b128, lane l: row l % 16, chunk 4 sub + l / 16) free of bank
//     conflicts. The loads of pair p + 2 go into the slot of pair p - 1,
//     half in each stage of pair p.
//   B ring: four slots of one stage (32 k rows of 256 n, 512 bytes each:
//     whole lines), 16 KiB each, laid out as 8 groups of 4 consecutive k rows,
//     2 KiB per group. Inside group G the 64-byte piece (32 n values) of k row
//     e in 32-wide n block s sits at byte (4 s + e) * 64, and its two 32-byte
//     halves (16 n values each) are swapped when bit 1 of G is set. Fragments
//     are read with ds_read_b64_tr_b16, which hands lane i of each 16-lane
//     group element i % 4 of the 8 bytes addressed by lane 4 e + i / 4 as its
//     element e: pointing lane 4 e + q at k row k0 + e, n n0 + 4 q gives lane
//     i the values (n n0 + i, k k0 .. k0 + 3); two such reads (groups 2 g and
//     2 g + 1) give the 8 k of a fragment. The two 16-lane groups of a half
//     wave read the same 16 columns of groups 2 g and 2 g + 2 (g = 0, 1),
//     whose swapped halves put them on disjoint banks: 256 bytes over all 64
//     banks, no conflicts. The loads of stage t + 4 go into the slot of stage
//     t, free once the barrier that starts stage t has passed.
//
// MFMA 16x16x32 bf16 register layout (lane l of 64, g = l / 16):
//   A fragment: row  l % 16, k = 8 g + [0..7] (16-byte chunk g of the stage)
//   B fragment: col  l % 16, k = 8 g + [0..7]
//   D (4 fp32): col  l % 16, row = 4 g + r
// (The k order inside a fragment only has to agree between A and B.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 32;         // k per stage
constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;  // voffset beyond every record count
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// A ring (K-major pairs)
constexpr int kPairK = 2 * kBK;                      // 64 k per pair
constexpr int kARowBytes = kPairK * 2;               // 128
constexpr int kAChunks = kARowBytes / 16;            // 8
constexpr int kASlotBytes = kBM * kARowBytes;        // 32 KiB
constexpr int kARowsPerLoad = 1024 / kARowBytes;     // 8
constexpr int kALoadsPerWavePair = (kBM / 4) / kARowsPerLoad;  // 8
constexpr int kASlots = 3;

// B ring (MN-major stages)
constexpr int kMnRowBytes = kBN * 2;                 // 512: one k row of 256 n values
constexpr int kMnGroupBytes = 4 * kMnRowBytes;       // 2 KiB: 4 interleaved k rows
constexpr int kMnPieceBytes = 64;                    // 32 n values of one k row
constexpr int kBSlotBytes = kBK * kMnRowBytes;       // 16 KiB
constexpr int kBLoadsPerWaveStage = kBK / 4 / 4 * 2;  // 4
constexpr int kBSlots = 4;

constexpr int kLoadsPerWaveStage = kALoadsPerWavePair / 2 + kBLoadsPerWaveStage;  // 8
constexpr int kLdsBytes = kASlots * kASlotBytes + kBSlots * kBSlotBytes;          // 160 KiB
static_assert(kLdsBytes == 160 * 1024, "the rings fill the CU's LDS");

// Byte offset of (row, 16-byte chunk) inside one A slot.
__device__ __forceinline__ int a_lds_off(int row, int chunk) {
  return (row * kAChunks + (chunk ^ ((row >> 1) & (kAChunks - 1)))) * 16;
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

// A workgroup barrier that orders LDS accesses only. __syncthreads() also
// fences global memory, so it waits for every vector-memory operation the
// wave has in flight (epilogue stores, the tile-queue atomic). The tile
// kernels pass data between waves through LDS alone, and direct-to-LDS
// loads are waited for explicitly (vmcnt) before their slots are read or
// reused.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// This thread's lane and wave, opaque to the optimiser. Per-tile setup derives
// many per-lane values (load offsets, epilogue indices) that do not depend on
// the tile; hoisted out of a persistent tile loop they stay live across the
// main loop, which needs nearly every register, and get spilled to scratch
// and reloaded every tile. Reading the lane through an empty asm inside the
// loop keeps them per tile: a few VALU instructions instead of scratch traffic.
__device__ __forceinline__ int lane_fresh() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}
// A wave-uniform value the compiler cannot see through, so nothing derived
// from it is computed ahead of the point where it is produced.
__device__ __forceinline__ int sgpr_fresh(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ int wave_fresh() {
  int w = threadIdx.x >> 6;
  asm volatile("" : "+v"(w));
  return w;
}

// A buffer descriptor must live in SGPRs: its inputs go through readfirstlane
// so the compiler sees them as wave-uniform (they are uniform by design).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The K-major A operand of a tile: rows m0 .. m0 + 255 of a [rows][ld] bf16
// matrix; rows at or past `rows` (counted from m0) read as zero.
//
// Each wave loads 64 of the 256 rows, so each wave builds its descriptor at
// its own first row: record counts and lane offsets then span at most
// 64 rows, 128 ld bytes, which stays below 2^31 (and below the kOOB
// sentinel) for every ld < 2^24. A descriptor over the whole tile would
// span 512 ld bytes and wrap at ld = 2^22.
constexpr int64_t kMaxALd = int64_t(1) << 24;
struct ASrc {
  __amdgpu_buffer_rsrc_t rsrc;
  __amdgpu_buffer_rsrc_t none;         // zero records: every load reads zeros
  uint32_t off[kALoadsPerWavePair];   // per load: byte offset of this lane's chunk at k = 0

  // tile_base: element pointer of the tile's first row; ld: row pitch
  // (elements, multiple of 8, below kMaxALd; every row holds the K range
  // rounded up to 64).
  __device__ __forceinline__ void init(const uint16_t* tile_base, int64_t ld, int rows) {
    const int lane = lane_fresh();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int kWaveRows = kBM / 4;
    int wrows = rows - wave * kWaveRows;  // rows of this wave's 64 that exist
    wrows = wrows < 0 ? 0 : (wrows > kWaveRows ? kWaveRows : wrows);
    const int bytes = __builtin_amdgcn_readfirstlane((int)((int64_t)wrows * ld * 2));
    void* base = reinterpret_cast<void*>(
        uniform_u64(reinterpret_cast<uint64_t>(tile_base + (int64_t)wave * kWaveRows * ld)));
    rsrc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kRsrcWord3);
    none = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < kALoadsPerWavePair; ++j) {
      const int wr = j * kARowsPerLoad + lane / kAChunks;  // row within the wave's 64
      // the LDS swizzle follows the row within the tile; wave * 64 leaves
      // (row >> 1) & 7 unchanged
      const int c = (lane % kAChunks) ^ ((wr >> 1) & (kAChunks - 1));
      off[j] = wr < wrows ? (uint32_t)(wr * ld * 2 + c * 16) : kOOB;
    }
  }
  // Issue load j (0..7) of this wave's loads of k pair p into the A slot at
  // `dst`; pairs at or past np read as zeros.
  __device__ __forceinline__ void issue_one(int p, int np, int j, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* base = dst + wave * (kBM / 4) * kARowBytes;
    // the k offset rides in the scalar soffset field; rows past the end keep
    // voffset >= the record count whether or not soffset enters the check
    const bool live = p < np;
    const int koff = __builtin_amdgcn_readfirstlane(live ? p * kARowBytes : 0);
    const __amdgpu_buffer_rsrc_t r = live ? rsrc : none;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + j * 1024), 16, off[j], koff, 0,
                                             0);
  }
  __device__ __forceinline__ void issue_pair(int p, int np, char* dst) const {
#pragma unroll
    for (int j = 0; j < kALoadsPerWavePair; ++j) issue_one(p, np, j, dst);
  }
  // Fragment of stage `sub` (0, 1) of the pair, 16-row block i (0..7) of the
  // wave's 128-row half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* slot, int sub, int lane, int half,
                                                  int i) {
    // the swizzle depends on lane & 15 only: 16-row blocks start at rows
    // that are multiples of 16
    const int o = a_lds_off(lane & 15, 4 * sub + (lane >> 4));
    return *reinterpret_cast<const bf16x8_t*>(slot + (half * 128 + i * 16) * kARowBytes + o);
  }
};

// The MN-major B operand of a tile: columns n0 .. n0 + 255 of the k rows of a
// [k_rows][ld] bf16 matrix (n contiguous); k rows at or past k_rows and
// columns at or past n_valid (counted from n0) read as zero.
//
// Each wave loads 8 of a stage's 32 k rows, and its descriptor starts at its
// own first row of the stage: record counts and offsets span at most 8 rows,
// 16 ld bytes, below 2^31 for every ld < 2^27.
constexpr int64_t kMaxBLd = int64_t(1) << 27;
struct BSrc {
  uint64_t base;                        // byte address of (k = 8 wave, n0); wave-uniform
  int64_t pitch;                        // bytes per k row; wave-uniform
  int k_valid;                          // k rows at or past the wave's first; wave-uniform
  uint32_t off[kBLoadsPerWaveStage];   // per load: byte offset of this lane's chunk in a stage

  __device__ __forceinline__ void init(const uint16_t* col_base, int64_t ld, int k_rows,
                                       int n_valid) {
    constexpr int kWaveRows = kBK / 4;  // 8 k rows of each stage per wave
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    base = uniform_u64(reinterpret_cast<uint64_t>(col_base + (int64_t)wave * kWaveRows * ld));
    pitch = (int64_t)uniform_u64((uint64_t)(ld * 2));
    k_valid = __builtin_amdgcn_readfirstlane((k_rows < 0 ? 0 : k_rows) - wave * kWaveRows);
    const int lane = lane_fresh();
    const int e = (lane >> 2) & 3;     // k row inside the group
    const int blk = lane >> 4;         // 32-wide n block inside the half
    // 16-byte chunk inside the piece: the wave fills groups 2 wave and
    // 2 wave + 1, whose bit 1 is wave & 1; there the 32-byte halves swap
    const int cq = (lane & 3) ^ ((wave & 1) << 1);
#pragma unroll
    for (int j = 0; j < kBLoadsPerWaveStage; ++j) {
      // load j fills half (j & 1) of group 2 wave + j / 2 of the stage; its
      // k row relative to the wave's first row of the stage:
      const int row = (j >> 1) * 4 + e;
      const int col = ((j & 1) * 4 + blk) * 32 + cq * 8;
      off[j] = col < n_valid ? (uint32_t)(row * pitch + col * 2) : kOOB;
    }
  }
  // The descriptor of this wave's loads of stage kt: rebased to the wave's
  // first k row of the stage, its record count covering only the valid rows
  // among the wave's 8 (none at or past k_rows).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(int kt) const {
    constexpr int kWaveRows = kBK / 4;
    int rows = k_valid - kt * kBK;
    rows = rows < 0 ? 0 : (rows > kWaveRows ? kWaveRows : rows);
    void* p = reinterpret_cast<void*>(uniform_u64(base + (uint64_t)((int64_t)kt * kBK * pitch)));
    const int bytes = __builtin_amdgcn_readfirstlane((int)(rows * pitch));
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes, kRsrcWord3);
  }
  // Issue load j (0..3) of a stage with descriptor r into the B slot at `dst`.
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t r, int j, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* ldsb = dst + wave * 2 * kMnGroupBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_ptr_t)(ldsb + (j >> 1) * kMnGroupBytes + (j & 1) * 1024), 16, off[j], 0, 0, 0);
  }
  __device__ __forceinline__ void issue(int kt, char* dst) const {
    const __amdgpu_buffer_rsrc_t r = stage_rsrc(kt);
#pragma unroll
    for (int j = 0; j < kBLoadsPerWaveStage; ++j) issue_one(r, j, dst);
  }
  static __device__ __forceinline__ bf16x4_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(lds_ptr_t)(p));
  }
  // Fragment of 16-column block j (0..7) of the wave's 128-column half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* slot, int lane, int half, int j) {
    // lane 16 g + 4 e + q reads k rows 8 g + e (group 2 g) and 8 g + 4 + e
    // (group 2 g + 1) at n = 128 half + 16 j + 4 q: 32-wide block
    // 4 half + j / 2, 32-byte half (j & 1) ^ (g & 1) of the piece
    const int g = lane >> 4;
    const int lane_part = g * 2 * kMnGroupBytes + ((lane >> 2) & 3) * kMnPieceBytes +
                          (((j & 1) ^ (g & 1)) << 5) + (lane & 3) * 8;
    const char* p = slot + (half * 4 + (j >> 1)) * 4 * kMnPieceBytes + lane_part;
    const bf16x4_t lo = tr_read(p);
    const bf16x4_t hi = tr_read(p + kMnGroupBytes);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// ---------------------------------------------------------------------------
// Tile scheduling: persistent workgroups, XCD-aware grouped order.
// Workgroups are dispatched round-robin over the 8 XCDs (chiplets), 32 per
// XCD at full occupancy. Each round of `grid` logical tiles is dealt to the
// XCDs in blocks of grid / 8 consecutive tiles (TileQueue below); logical
// tiles run in groups of GM m-tiles by all n-tiles (m fastest inside a
// group), so the 32 concurrent tiles of an XCD form a GM x (32 / GM) block
// sharing A and B panels in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
// Group widths (m-tiles per group) of each GEMM; a group is swept with m
// fastest, so an XCD's 32 concurrent tiles cover gm m-tiles by 32 / gm n-tiles
// and read gm + 32 / gm operand panels (12 for gm = 4 or 8, the fewest). Timed
// per GEMM with widths 4, 8 and 16 on three batches (N 16384 with H 4096 /
// V 131072, H 4096 / V 151936 and H 2560 / V 151936): 16 is slower for every
// GEMM; 8 is best or tied for fwd, dz and dW; dX is 0.4-1.1 % faster with 4.
#ifndef LMH_GM_FWD
#define LMH_GM_FWD 8
#endif
#ifndef LMH_GM_DZ
#define LMH_GM_DZ 8
#endif
#ifndef LMH_GM_DX
#define LMH_GM_DX 4
#endif
#ifndef LMH_GM_DW
#define LMH_GM_DW 8
#endif

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

// Dynamic tile queues. Logical tiles are dealt to the XCDs as in the static
// order above (the per = grid / 8 workgroups of an XCD take consecutive
// logical tiles of each round), but each XCD hands its tiles out from its own
// counter in device memory, and with `steal` a workgroup whose XCD has none
// left takes the next tile of another XCD's queue. The XCDs do not run at the
// same speed under these kernels (measured: up to 4 % apart), so with a fixed
// assignment the slowest one sets the kernel time; stealing only pays when a
// tile is a small part of a workgroup's work, so the host enables it for
// launches with many tiles per workgroup.
__device__ __forceinline__ int xcd_id() {
  // s_getreg_b32 hwreg(HW_REG_XCC_ID, 0, 4): the XCD this wave runs on
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (kXcds - 1);
}

struct TileQueue {
  int* ctr;    // [kXcds] counters, zero before the launch
  int ntiles;  // logical tiles of this launch
  int steal;
  int ahead;   // thread 0: counter value taken by claim_ahead, or kNone
  static constexpr int kNone = -1;

  __device__ TileQueue(int* c, int n, int st) : ctr(c), ntiles(n), steal(st), ahead(kNone) {}

  // Thread 0: takes the next position of XCD y's counter. An increment, not
  // an add: the compiler rewrites a lone lane's add into a wave-wide form
  // that waits for the result on the spot.
  __device__ __forceinline__ int take(int y) const {
    return (int)atomicInc(reinterpret_cast<unsigned*>(&ctr[y]), 0xffffffffu);
  }
  // The tile at position k of XCD y's queue, or -1 past its end.
  __device__ __forceinline__ int tile_at(int y, int k) const {
    const int grid = gridDim.x;
    const int per = grid / kXcds;
    const int full = ntiles / grid, rem = ntiles - full * grid;
    const int count = full * per + min(per, max(0, rem - per * y));
    return k < count ? (k / per) * grid + y * per + k % per : -1;
  }

  // Called by every thread once a tile's main loop is done: thread 0 takes
  // the next position of its own XCD's queue now, so that the atomic's
  // latency is hidden under the epilogue.
  __device__ __forceinline__ void claim_ahead() {
    if (threadIdx.x == 0) ahead = take(xcd_id());
  }

  // The next logical tile for the calling workgroup, or -1 when none is left.
  // Thread 0 takes it (the position taken ahead, else the next one of its
  // own XCD's queue, then the other queues when stealing) and broadcasts it
  // through the first word of `bcast`, the ring slot bcast_slot<SHIFT>()
  // names (no load writes it until every wave has read the index); contains
  // a workgroup barrier (LDS only: the atomics are thread 0's own).
  __device__ __forceinline__ int next(char* bcast) {
    // an LDS pointer, so the exchange is a ds_write / ds_read pair (through a
    // generic pointer it is a flat access, which also waits for the stores
    // of the epilogue before it)
    volatile __attribute__((address_space(3))) int* slot =
        (volatile __attribute__((address_space(3))) int*)bcast;
    if (threadIdx.x == 0) {
      const int x = xcd_id();
      int t = tile_at(x, ahead != kNone ? ahead : take(x));
      ahead = kNone;
      for (int d = 1; t < 0 && steal && d < kXcds; ++d) {
        const int y = (x + d) & (kXcds - 1);
        t = tile_at(y, take(y));
      }
      *slot = t;
    }
    lds_barrier();
    return *slot;
  }
};

// ---------------------------------------------------------------------------
// Main loop.
// ---------------------------------------------------------------------------
// The ring slot through whose first word thread 0 hands the next tile index
// to the workgroup (TileQueue::next). The main loop's prologue loads B slots
// SHIFT, SHIFT + 1 and SHIFT + 2 (mod 4) and both A slots of pairs 0 and 1
// before its first barrier; B slot SHIFT + 3 is loaded only after it, by
// which point every wave has read the index. Epilogues stage through A slots
// only. (Only wave 0 writes the first bytes of any slot, and its loads have
// landed when a main loop returns.)
template <int SHIFT>
__host__ __device__ constexpr int bcast_slot() { return (SHIFT + 3) % 4; }

struct Ring {
  char* a[3];
  char* b[4];
};

// The ring slots must be distinct __shared__ objects named at every access
// (see mainloop); kernels declare them with this macro, which also defines
// `ring`.
#define LMH_DECLARE_RING                                                   \
  __shared__ __attribute__((aligned(1024))) char ra0[lmh::kASlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char ra1[lmh::kASlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char ra2[lmh::kASlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char rb0[lmh::kBSlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char rb1[lmh::kBSlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char rb2[lmh::kBSlotBytes];    \
  __shared__ __attribute__((aligned(1024))) char rb3[lmh::kBSlotBytes];    \
  const lmh::Ring ring = {{ra0, ra1, ra2}, {rb0, rb1, rb2, rb3}}

// The fragments of one stage: A blocks a[i] (16 rows each) and B blocks b[j]
// (16 columns each) of the wave's 128 x 128 sub-tile.
struct Frags {
  bf16x8_t a[8], b[8];
};

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef f32x4_t Acc[8][8];  // the wave's accumulators, block (i, j) at acc[i][j]

// Fragments of the stage held in A slot `as` (stage `sub` of its pair) and
// B slot `bs`. B and A reads alternate so that the slower transposing reads
// start early.
__device__ __forceinline__ void read_frags(const char* as, int sub, const char* bs, int lane,
                                           int wm, int wn, Frags& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f.b[j] = BSrc::frag(bs, lane, wn, j);
    f.a[j] = ASrc::frag(as, sub, lane, wm, j);
  }
}

// One MFMA accumulating in place into the AGPR quad that holds c. The
// builtin form lets the compiler pick a separate destination quad, and with
// 64 accumulators filling the AGPRs it then shuttles results through vector
// registers (hundreds of copies per stage); tied in place, every accumulator
// keeps its quad. The compiler does not see this as an MFMA, so it inserts no
// hazard waits for it: an accumulator is used again only 64 MFMAs later, and
// acc_fence (below) separates the last MFMA from any other read.
__device__ __forceinline__ void mfma16(f32x4_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Every accumulator quad of the wave as an in/out AGPR operand of an asm
// statement.
#define LMH_ACC_OPERANDS(c) \
    "+a"(c[0][0]), "+a"(c[0][1]), "+a"(c[0][2]), "+a"(c[0][3]), "+a"(c[0][4]), \
    "+a"(c[0][5]), "+a"(c[0][6]), "+a"(c[0][7]), "+a"(c[1][0]), "+a"(c[1][1]), \
    "+a"(c[1][2]), "+a"(c[1][3]), "+a"(c[1][4]), "+a"(c[1][5]), "+a"(c[1][6]), \
    "+a"(c[1][7]), "+a"(c[2][0]), "+a"(c[2][1]), "+a"(c[2][2]), "+a"(c[2][3]), \
    "+a"(c[2][4]), "+a"(c[2][5]), "+a"(c[2][6]), "+a"(c[2][7]), "+a"(c[3][0]), \
    "+a"(c[3][1]), "+a"(c[3][2]), "+a"(c[3][3]), "+a"(c[3][4]), "+a"(c[3][5]), \
    "+a"(c[3][6]), "+a"(c[3][7]), "+a"(c[4][0]), "+a"(c[4][1]), "+a"(c[4][2]), \
    "+a"(c[4][3]), "+a"(c[4][4]), "+a"(c[4][5]), "+a"(c[4][6]), "+a"(c[4][7]), \
    "+a"(c[5][0]), "+a"(c[5][1]), "+a"(c[5][2]), "+a"(c[5][3]), "+a"(c[5][4]), \
    "+a"(c[5][5]), "+a"(c[5][6]), "+a"(c[5][7]), "+a"(c[6][0]), "+a"(c[6][1]), \
    "+a"(c[6][2]), "+a"(c[6][3]), "+a"(c[6][4]), "+a"(c[6][5]), "+a"(c[6][6]), \
    "+a"(c[6][7]), "+a"(c[7][0]), "+a"(c[7][1]), "+a"(c[7][2]), "+a"(c[7][3]), \
    "+a"(c[7][4]), "+a"(c[7][5]), "+a"(c[7][6]), "+a"(c[7][7])

// The compiler treats the asm MFMAs as opaque, so it cannot honour their
// hazards: a VALU write of an accumulator (its zeroing) must not be placed
// right before the first MFMA that reads it, and no read may follow the last
// MFMA too closely. acc_pin, after the zeroing, makes every accumulator live
// in its AGPR at that point; being volatile it stays ahead of the main loop's
// prologue (loads, barrier, fragment reads), which keeps the zeroing writes
// far from the first MFMAs. (Sunk next to their MFMAs they corrupted the
// first and last register of some quads.)
__device__ __forceinline__ void acc_pin(Acc& c) { asm volatile("" : LMH_ACC_OPERANDS(c)); }

// 24 wait states, more than an MFMA's write-to-read distance, depending on
// every accumulator: no read of an accumulator (ours or the compiler's) can be
// placed between the main loop's last MFMAs and this.
__device__ __forceinline__ void acc_fence(Acc& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : LMH_ACC_OPERANDS(c));
}

constexpr int kMfmaPerStage = 64;
// The stage's MFMAs run A block by A block (row i of the wave's 8 x 8
// blocks), the B blocks of odd rows in reverse, so that consecutive MFMAs
// change one operand only (the row's last B block starts the next row). The
// chip's clock under MFMA load falls with the operand bits that switch from
// one MFMA to the next: with the bench batch's operands in registers this
// order ran 1.0 % faster than every row in ascending order, at a 1 % higher
// clock. Each accumulator still sums its k steps in the same order.
__host__ __device__ constexpr int mfma_col(int m) {
  return ((m / 8) & 1) ? 7 - m % 8 : m % 8;
}
// The next stage's fragment reads go out as 16 units (B block u / 2 -- two
// transposing reads -- for even u, A block u / 2 for odd u), unit u after
// MFMA (7 u) / 2: spread over the first 53 MFMAs so that the last reads land
// well before the next barrier. The slower transposing reads go first.
constexpr int kReadUnits = 16;
__host__ __device__ constexpr int read_slot(int u) { return (7 * u) / 2; }
__host__ __device__ constexpr int read_unit_at(int m) {
  const int u = (2 * m + 6) / 7;  // the one unit whose slot can be m
  return (u < kReadUnits && read_slot(u) == m) ? u : -1;
}
__host__ __device__ constexpr int count_read_slots() {
  int n = 0;
  for (int m = 0; m < 64; ++m) n += read_unit_at(m) >= 0;
  return n;
}
static_assert(count_read_slots() == kReadUnits && read_slot(kReadUnits - 1) < kMfmaPerStage,
              "every read unit has exactly one MFMA slot");
// The stage's 8 loads go out after MFMAs 4, 12, .., 60: A loads first, then B.
__host__ __device__ constexpr int load_at(int m) { return m % 8 == 4 ? m / 8 : -1; }

// Stage t (U = t + SHIFT mod 12, a compile-time stage of the 12-stage
// period, so every slot index below is a compile-time constant). On entry
// `cur` holds stage t's fragments (read during stage t - 1) and stage t + 1's
// operands are landing. Every wave waits for its loads of stage t + 1 and for
// its fragment reads of stage t; the barrier then publishes stage t + 1 and
// releases stage t's B slot (and, after the pair's second stage, its A slot).
// The 64 MFMAs of stage t run on `cur` while stage t + 1's fragments are read
// into `nxt`, half of pair t / 2 + 2's A loads go into the slot pair
// t / 2 - 1 released, and stage t + 4's B loads go into stage t's slot. The
// order is fixed by hand (sched_barrier after every MFMA): the compiler's
// scheduler does not see the asm MFMAs as MFMAs.
//
// Loads issued per stage, in order: 4 of A, then 4 of B. At the start of
// stage t the loads needed are B stage t + 1 (issued in stage t - 3) and,
// when t + 1 starts a pair, that pair's second half (issued in stage t - 2,
// before its B loads); the loads issued after them number 16 (t even) or
// 12 (t odd).
template <int U>
__device__ __forceinline__ void k_stage(const ASrc& A, const BSrc& B, int t, int np,
                                        const Ring& R, int lane, int wm, int wn, Frags& f0,
                                        Frags& f1, Acc& acc) {
  static_assert(kLoadsPerWaveStage == 8, "the waits below assume 8 loads per stage");
  constexpr int a_nxt = ((U + 1) / 2) % 3, sub_nxt = (U + 1) % 2;
  constexpr int a_fre = (U / 2 + 2) % 3, b_nxt = (U + 1) % 4, b_fre = U % 4;
  Frags& cur = (U % 2) ? f1 : f0;
  Frags& nxt = (U % 2) ? f0 : f1;
  wait_vmcnt<(U % 2) ? 12 : 16>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const __amdgpu_buffer_rsrc_t brs = B.stage_rsrc(t + 4);
  const int pair = t / 2 + 2;
#pragma unroll
  for (int m = 0; m < kMfmaPerStage; ++m) {
    const int i = m / 8, j = mfma_col(m);
    mfma16(acc[i][j], cur.a[i], cur.b[j]);
    const int q = load_at(m);
    if (q >= 0 && q < 4) A.issue_one(pair, np, (U % 2) * 4 + q, R.a[a_fre]);
    if (q >= 4) B.issue_one(brs, q - 4, R.b[b_fre]);
    const int u = read_unit_at(m);
    if (u >= 0 && u % 2 == 0) nxt.b[u / 2] = BSrc::frag(R.b[b_nxt], lane, wn, u / 2);
    if (u >= 0 && u % 2 == 1) nxt.a[u / 2] = ASrc::frag(R.a[a_nxt], sub_nxt, lane, wm, u / 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Accumulates the tile over nk stages of kBK. The caller must have made the
// LDS free (barrier) before the call; on return every wave has finished its
// LDS reads and no load is in flight. The slots are distinct __shared__
// objects and the loop is unrolled by 12 (the periods of the two rings are
// 6 and 4 stages, of the fragment sets 2), so every LDS access names a fixed
// slot: the compiler can then see that fragment reads never alias the
// direct-to-LDS loads in flight into other slots, and inserts no waits of
// its own.
//
// SHIFT (even, 0..10) starts the slot rotation at virtual stage SHIFT: the
// first 12 - SHIFT stages run as straight-line copies of bodies SHIFT..11
// before the loop, so a stage count with nk + SHIFT a multiple of 12 runs no
// padding stage. Any other count runs up to 11 stages past nk, which read
// zeros and add nothing (an early exit instead would be a branch out of the
// unrolled body, and any such branch makes the register allocator spill
// fragments inside the loop). nk <= 0 is allowed and yields zeros.
template <int SHIFT = 0>
__device__ __forceinline__ void mainloop(const ASrc& A, const BSrc& B, int nk, const Ring& R,
                                         Acc& acc) {
  static_assert(SHIFT % 2 == 0 && SHIFT >= 0 && SHIFT < 12, "A pairs must stay aligned");
  constexpr int kPeel = (12 - SHIFT) % 12;
  // fresh per call: the fragment addresses derived from them are computed per
  // tile instead of being kept (and spilled) across the epilogues
  const int lane = lane_fresh();
  const int wave = wave_fresh();
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int np = (nk + 1) / 2;  // nk <= 0: the prologue's loads read zeros

  // Prologue: pairs 0 and 1, stages 0..3. Stage 3 goes into the B slot that
  // carries the tile index (bcast_slot) and so only after the first barrier.
  constexpr int a0 = (SHIFT / 2) % 3, a1 = (SHIFT / 2 + 1) % 3;
  constexpr int b0 = SHIFT % 4, b1 = (SHIFT + 1) % 4, b2 = (SHIFT + 2) % 4, b3 = (SHIFT + 3) % 4;
  static_assert(b3 == bcast_slot<SHIFT>(), "the tile-index slot is loaded after the barrier");
  A.issue_pair(0, np, R.a[a0]);
  B.issue(0, R.b[b0]);
  B.issue(1, R.b[b1]);
  A.issue_pair(1, np, R.a[a1]);
  B.issue(2, R.b[b2]);
  // the accumulators are zeroed while those loads are in flight (256 VALU
  // writes, hidden under their latency)
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  acc_pin(acc);
  // (nk <= 0 takes no early exit: a branch here makes the register allocator
  // spill; the peel stages below then run over zero-filled loads)
  // pair 0 and stage 0 landed: only stage 1, pair 1 and stage 2 may remain
  wait_vmcnt<2 * kBLoadsPerWaveStage + kALoadsPerWavePair>();
  __builtin_amdgcn_s_barrier();
  B.issue(3, R.b[b3]);

  Frags f0, f1;
  // stage 0 is fragment set SHIFT % 2 = 0
  read_frags(R.a[a0], 0, R.b[b0], lane, wm, wn, f0);
  if constexpr (kPeel > 0) {
#define LMH_PEEL(U) \
  if constexpr (U >= SHIFT) k_stage<U>(A, B, sgpr_fresh(U - SHIFT), np, R, lane, wm, wn, f0, f1, acc);
    LMH_PEEL(0) LMH_PEEL(1) LMH_PEEL(2) LMH_PEEL(3) LMH_PEEL(4) LMH_PEEL(5)
    LMH_PEEL(6) LMH_PEEL(7) LMH_PEEL(8) LMH_PEEL(9) LMH_PEEL(10) LMH_PEEL(11)
#undef LMH_PEEL
  }
  for (int s = kPeel; s < nk; s += 12) {
#define LMH_STAGE(U) k_stage<U>(A, B, s + U, np, R, lane, wm, wn, f0, f1, acc);
    LMH_STAGE(0) LMH_STAGE(1) LMH_STAGE(2) LMH_STAGE(3) LMH_STAGE(4) LMH_STAGE(5)
    LMH_STAGE(6) LMH_STAGE(7) LMH_STAGE(8) LMH_STAGE(9) LMH_STAGE(10) LMH_STAGE(11)
#undef LMH_STAGE
  }
  // stages and pairs past the end issued loads and fragment reads that
  // nobody uses; let them land
  wait_vmcnt<0>();
  wait_lgkm0();
  acc_fence(acc);
}

// Epilogue reads of the accumulators. The compiler, left to itself, copies
// every accumulator block to vector registers right after the main loop (the
// copies land in the loop's exit block, ahead of the epilogue's branches),
// which fills the register file and serialises the epilogue. acc_read moves
// one accumulator register where its value is used. Every acc_read takes the
// token of an acc_read_fence issued after the main loop, so none is scheduled
// above it; the main loop itself ends with acc_fence, which keeps every read
// of an accumulator the MFMA write-to-read distance away from the last MFMA.
__device__ __forceinline__ int acc_read_fence() {
  int tok;
  asm volatile("s_mov_b32 %0, 0" : "=s"(tok) : : "memory");
  return tok;
}
__device__ __forceinline__ float acc_read(float x, int tok) {
  float y;
  asm("v_accvgpr_read_b32 %0, %1 ; after fence %2" : "=v"(y) : "a"(x), "s"(tok));
  return y;
}

// The SHIFT that makes nk (even) stages run without padding.
__host__ __device__ constexpr int stage_shift(int nk) { return (12 - nk % 12) % 12; }

// Row (within the wave's 128-row half) held by accumulator register r of
// block i: acc_row_fixed(i, r) + acc_row_lane(lane). Epilogues compare the
// compile-time part against a per-tile lane bound, so the compiler has no
// per-register lane values to keep live across the tile loop.
__host__ __device__ constexpr int acc_row_fixed(int i, int r) { return i * 16 + r; }
__device__ __forceinline__ int acc_row_lane(int lane) { return 4 * (lane >> 4); }

}  // namespace lmh
