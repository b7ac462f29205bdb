// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A[m][k] * B[n][k] with v_mfma_f32_32x32x16_bf16.
// Each wave owns a 128 x 128 sub-tile held as 4 x 4 MFMA accumulator blocks
// (256 AGPRs).
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
// kBK = 32; each stage issues four loads per wave for each operand, spread
// over the stage's MFMAs (one load per four MFMAs): a CU moves about 150 GB/s
// through these loads, twice what its MFMAs consume on average, so loads
// bunched into part of a stage stall the issuing wave. One barrier per stage
// publishes stage k + 1 and releases the LDS of stage k - 1. MFMA fragments
// are double-buffered in registers: the fragments of the next 16-wide k step
// are read from LDS while the current step's 16 MFMAs issue.
//
// LDS (160 KiB, all of it):
//   A ring: three slots of one k pair (64 k, two stages), 32 KiB each. A row
//     of the pair is 128 bytes, one whole L2 line: fetching K-major rows 64
//     bytes at a time would split every line across two requests, and the L2
//     fetches each 64-byte sector on its own miss. The 16-byte chunk index
//     is XOR-swizzled with (row >> 1) & 7, which keeps the fragment reads
//     (ds_read_b128, lane l: row l % 32, chunk 2 kq + l / 32) free of bank
//     conflicts. The loads of pair p + 2 go into the slot pair p - 1
//     released, half in each stage of pair p.
//   B ring: four slots of one stage (32 k rows of 256 n, 512 bytes each:
//     whole lines), 16 KiB each, laid out as 8 groups of 4 consecutive k rows,
//     2 KiB per group. Inside a group the 64-byte piece (32 n values) of k row
//     e in 32-wide n block s sits at byte (4 s + e) * 64. Fragments are read
//     with ds_read_b64_tr_b16, which hands lane i of each 16-lane group element
//     i % 4 of the 8 bytes addressed by lane 4 e + i / 4 as its element e:
//     pointing lane 4 e + q at k row k0 + e, n n0 + 4 q gives lane i the
//     values (n n0 + i, k k0 .. k0 + 3), the MFMA fragment shape; two such
//     reads give the 8 k of a fragment. A half wave reads 4 whole pieces that
//     are adjacent in LDS (256 contiguous bytes): no bank conflicts. The loads
//     of stage k + 3 go into the slot stage k - 1 released.
// A transpose read moves half the bytes of a ds_read_b128 in about the same
// LDS time, so the engine reads one operand (A) with ds_read_b128.
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
  // Issue half h (loads 4 h .. 4 h + 3) of this wave's loads of k pair p into
  // the A slot at `dst`; pairs at or past np read as zeros.
  __device__ __forceinline__ void issue_half(int p, int np, int h, char* dst) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* base = dst + wave * (kBM / 4) * kARowBytes;
    // the k offset rides in the scalar soffset field; rows past the end keep
    // voffset >= the record count whether or not soffset enters the check
    const bool live = p < np;
    const int koff = __builtin_amdgcn_readfirstlane(live ? p * kARowBytes : 0);
    const __amdgpu_buffer_rsrc_t r = live ? rsrc : none;
#pragma unroll
    for (int jj = 0; jj < kALoadsPerWavePair / 2; ++jj) {
      const int j = h * (kALoadsPerWavePair / 2) + jj;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + j * 1024), 16, off[j], koff,
                                               0, 0);
    }
  }
  // Fragment of 16-wide k step kq (0..3) of the pair, 32-row block i of the
  // wave's 128-row half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* slot, int kq, int lane, int half,
                                                  int i) {
    const int o = a_lds_off(lane & 31, kq * 2 + (lane >> 5));  // swizzle depends on lane & 31 only
    return *reinterpret_cast<const bf16x8_t*>(slot + (half * 128 + i * 32) * kARowBytes + o);
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
    const int cq = lane & 3;           // 16-byte chunk inside the piece
#pragma unroll
    for (int j = 0; j < kBLoadsPerWaveStage; ++j) {
      // load j fills half (j & 1) of group 2 wave + j / 2 of the stage; its
      // k row relative to the wave's first row of the stage:
      const int row = (j >> 1) * 4 + e;
      const int col = ((j & 1) * 4 + blk) * 32 + cq * 8;
      off[j] = col < n_valid ? (uint32_t)(row * pitch + col * 2) : kOOB;
    }
  }
  // Issue this wave's loads of stage kt into the B slot at `dst`. The
  // descriptor is rebased to the wave's first k row of the stage, and its
  // record count covers only the valid rows among the wave's 8 (none at or
  // past k_rows).
  __device__ __forceinline__ void issue(int kt, char* dst) const {
    constexpr int kWaveRows = kBK / 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* ldsb = dst + wave * 2 * kMnGroupBytes;
    int rows = k_valid - kt * kBK;
    rows = rows < 0 ? 0 : (rows > kWaveRows ? kWaveRows : rows);
    void* p = reinterpret_cast<void*>(uniform_u64(base + (uint64_t)((int64_t)kt * kBK * pitch)));
    const int bytes = __builtin_amdgcn_readfirstlane((int)(rows * pitch));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes,
                                                                       kRsrcWord3);
#pragma unroll
    for (int j = 0; j < kBLoadsPerWaveStage; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(ldsb + (j >> 1) * kMnGroupBytes + (j & 1) * 1024), 16, off[j], 0, 0, 0);
  }
  static __device__ __forceinline__ bf16x4_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(lds_ptr_t)(p));
  }
  // Fragment of k step kk (0..1) of the stage, 32-wide n block i of the
  // wave's 128 half `half`.
  static __device__ __forceinline__ bf16x8_t frag(const char* slot, int kk, int lane, int half,
                                                  int i) {
    // lane 16 g + 4 e + q reads k row 16 kk + 8 (g >> 1) + 4 h + e at n
    // 128 half + 32 i + 16 (g & 1) + 4 q, for the two halves h of the fragment
    const int g = lane >> 4;
    const int lane_part = (g >> 1) * 2 * kMnGroupBytes + ((lane >> 2) & 3) * kMnPieceBytes +
                          (g & 1) * 32 + (lane & 3) * 8;
    const char* p = slot + kk * 4 * kMnGroupBytes + (half * 4 + i) * 4 * kMnPieceBytes + lane_part;
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
  // a workgroup barrier.
  __device__ __forceinline__ int next(char* bcast) {
    volatile int* slot = reinterpret_cast<volatile int*>(bcast);
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
    __syncthreads();
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

struct Frags {
  bf16x8_t a[4], b[4];
};

// Fragments of one 16-wide k step: A data is k step kq (0..3) of the pair in
// slot `as`, B data is k step kk (0..1) of the stage in slot `bs`.
__device__ __forceinline__ void read_frags(const char* as, int kq, const char* bs, int kk,
                                           int lane, int wm, int wn, Frags& f) {
  // first-use order of mfma_step: a0 with b0..b3, then a1, a2, a3
  f.a[0] = ASrc::frag(as, kq, lane, wm, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = BSrc::frag(bs, kk, lane, wn, j);
#pragma unroll
  for (int i = 1; i < 4; ++i) f.a[i] = ASrc::frag(as, kq, lane, wm, i);
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
constexpr int kReadsPerStep = 4 * 1 + 4 * 2;  // A: one ds_read_b128, B: two transpose reads

// Interleaves the 16 MFMAs of a k step with its 12 LDS reads (one after each
// of the first 12 MFMAs) and its 4 loads (one per four MFMAs).
template <int ID>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, ID);
    if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, ID);
    if (i < kReadsPerStep) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, ID);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stage s = s0 + U of the main loop (s0 a multiple of 12, so every slot
// index below is a compile-time constant). On entry f0 holds stage s's
// kk = 0 fragments. Step 1 runs kk = 0 while reading kk = 1 into f1 and
// issuing half of pair s / 2 + 2's A loads (into the slot pair s / 2 - 1
// released). Then every wave waits for its loads of stage s + 1 (at most the
// 8 loads of stage s - 1 and the 4 just issued may remain) and for its LDS
// reads, and the barrier publishes stage s + 1 and releases stage s's B slot
// and, after the pair's second stage, its A slot. Step 2 runs kk = 1 while
// reading stage s + 1's kk = 0 fragments and issuing stage s + 3's B loads
// (into the slot stage s - 1 released).
template <int U>
__device__ __forceinline__ void k_stage(const ASrc& A, const BSrc& B, int s, int np,
                                        const Ring& R, int lane, int wm, int wn, Frags& f0,
                                        Frags& f1, f32x16_t (&acc)[4][4]) {
  static_assert(kLoadsPerWaveStage == 8, "the wait below assumes 8 loads per stage");
  constexpr int a_cur = (U / 2) % 3, a_nxt = ((U + 1) / 2) % 3, a_fre = (U / 2 + 2) % 3;
  constexpr int b_cur = U % 4, b_nxt = (U + 1) % 4, b_fre = (U + 3) % 4;
  constexpr int sub = U % 2, sub_nxt = (U + 1) % 2;
  __builtin_amdgcn_sched_barrier(0);
  read_frags(R.a[a_cur], 2 * sub + 1, R.b[b_cur], 1, lane, wm, wn, f1);
  A.issue_half(s / 2 + 2, np, sub, R.a[a_fre]);
  mfma_step(f0, acc);
  interleave<0>();
  wait_vmcnt<kLoadsPerWaveStage + kALoadsPerWavePair / 2>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(R.a[a_nxt], 2 * sub_nxt, R.b[b_nxt], 0, lane, wm, wn, f0);
  B.issue(s + 3, R.b[b_fre]);
  mfma_step(f1, acc);
  interleave<1>();
}

// Accumulates the tile over nk stages of kBK. The caller must have made the
// LDS free (barrier) before the call; on return every wave has finished its
// LDS reads and no load is in flight. The slots are distinct __shared__
// objects and the loop is unrolled by 12 (the periods of the two rings are
// 6 and 4 stages), so every LDS access names a fixed slot: the compiler can
// then see that fragment reads never alias the direct-to-LDS loads in flight
// into other slots, and inserts no waits of its own.
//
// SHIFT (even, 0..10) starts the slot rotation at virtual stage SHIFT: the
// first 12 - SHIFT stages run as straight-line copies of bodies SHIFT..11
// before the loop, so a stage count with nk + SHIFT a multiple of 12 runs no
// padding stage. Any other count runs up to 11 stages past nk, which read
// zeros and add nothing (an early exit instead would be a branch out of the
// unrolled body, and any such branch makes the register allocator spill
// fragments inside the loop).
template <int SHIFT = 0>
__device__ __forceinline__ void mainloop(const ASrc& A, const BSrc& B, int nk, const Ring& R,
                                         f32x16_t (&acc)[4][4]) {
  static_assert(SHIFT % 2 == 0 && SHIFT >= 0 && SHIFT < 12, "A pairs must stay aligned");
  constexpr int kPeel = (12 - SHIFT) % 12;
  // fresh per call: the fragment addresses derived from them are computed per
  // tile instead of being kept (and spilled) across the epilogues
  const int lane = lane_fresh();
  const int wave = wave_fresh();
  const int wm = wave >> 1;
  const int wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;
  const int np = (nk + 1) / 2;

  // Issue order matters: each stage's wait counts loads issued after the ones
  // it needs. At stage 0's wait, B stage 1 must be older than the last 12
  // loads (A pair 1's second half, B stage 2, pair 2's first half).
  constexpr int a0 = (SHIFT / 2) % 3, a1 = (SHIFT / 2 + 1) % 3;
  constexpr int b0 = SHIFT % 4, b1 = (SHIFT + 1) % 4, b2 = (SHIFT + 2) % 4;
  static_assert(b0 != bcast_slot<SHIFT>() && b1 != bcast_slot<SHIFT>() &&
                    b2 != bcast_slot<SHIFT>(),
                "the prologue must not load the tile-index slot before its first barrier");
  A.issue_half(0, np, 0, R.a[a0]);
  A.issue_half(0, np, 1, R.a[a0]);
  B.issue(0, R.b[b0]);
  B.issue(1, R.b[b1]);
  A.issue_half(1, np, 0, R.a[a1]);
  A.issue_half(1, np, 1, R.a[a1]);
  B.issue(2, R.b[b2]);
  // pair 0 and stage 0 landed: only stage 1, pair 1 and stage 2 may remain
  wait_vmcnt<kALoadsPerWavePair + 2 * kBLoadsPerWaveStage>();
  __builtin_amdgcn_s_barrier();

  Frags f0, f1;
  read_frags(R.a[a0], 0, R.b[b0], 0, lane, wm, wn, f0);
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
  // stages and pairs past the end issued loads that nobody reads; let them land
  wait_vmcnt<0>();
  wait_lgkm0();
}

// Epilogue reads of the accumulators. The compiler, left to itself, copies
// every accumulator block to vector registers right after the main loop (the
// copies land in the loop's exit block, ahead of the epilogue's branches),
// which fills the register file and serialises the epilogue. acc_read moves
// one accumulator register where its value is used. The hardware does not
// interlock an accumulator read on an MFMA still writing it, and the compiler
// does not see into the asm, so every acc_read takes the token of an
// acc_read_fence (24 wait states, more than the write-to-read distance of
// even a 16-pass MFMA) issued after the main loop: no read is scheduled
// above it.
__device__ __forceinline__ int acc_read_fence() {
  int tok;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_mov_b32 %0, 0" : "=s"(tok) : : "memory");
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
__host__ __device__ constexpr int acc_row_fixed(int i, int r) {
  return i * 32 + 8 * (r >> 2) + (r & 3);
}
__device__ __forceinline__ int acc_row_lane(int lane) { return 4 * (lane >> 5); }

}  // namespace lmh
