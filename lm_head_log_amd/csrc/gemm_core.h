// gemm_core.h - bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) computes a 256 x 256
// fp32 tile C[m][n] = sum_k A(m, k) * B(k, n) with v_mfma_f32_32x32x16_bf16.
// Each wave owns a 128 x 128 sub-tile held as 4 x 4 MFMA accumulator blocks.
// K advances in steps of 64 through a double-buffered LDS stage; the next
// stage's global loads are issued before the current stage's MFMAs.
//
// Operands are staged in LDS "K-inner": every tile row (an m for A, an n for B)
// stores its 64 k values as eight 16-byte chunks. A chunk's position in the row
// is XOR-swizzled with bits of the row index so that the three access patterns
// (MFMA fragment reads, row-contiguous staging writes, transposed staging
// writes) touch distinct LDS banks within every group of eight lanes.
//
// Two global layouts are supported per operand:
//   K-major  : the operand's rows are contiguous in k (X rows, W rows, dZ rows
//              when k = vocab). Staged with 16-byte loads and stores.
//   MN-major : k is the slow index (W when k = vocab in dX = dZ W; dZ and the
//              gathered X when k = token in dW = dZ^T X). Each thread loads an
//              8 x 8 bf16 block (8 rows of 16 bytes), transposes it in
//              registers (byte permutes), and writes eight 16-byte chunks.
//
// MFMA 32x32x16 bf16 register layout (lane l, 64 lanes):
//   A fragment: row  l % 32, k = 8 * (l / 32) + [0..7]
//   B fragment: col  l % 32, k = 8 * (l / 32) + [0..7]
//   D (16 fp32): col l % 32, row = 8 * (r / 4) + 4 * (l / 32) + (r % 4)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kStageChunks = kBM * (kBK / 8);  // 16-byte chunks per operand stage

// Swizzled chunk index of (row, chunk) inside a K-inner LDS stage.
__device__ __forceinline__ int lds_slot(int row, int chunk) {
  return row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// ---------------------------------------------------------------------------
// Operand stagers. Each thread owns 8 16-byte chunks of a 256 x 64 stage.
// ---------------------------------------------------------------------------

// K-major operand: tile row r (0..255) maps to global row g(r), k contiguous.
// Thread t stages chunk (t % 8) of tile rows t/8 + 32 j, j = 0..7.
struct KMajorStager {
  const uint4* ptr[8];
  uint32_t ok;  // bit j: row slot j is inside the matrix
  uint4 reg[8];

  // base: element pointer of row 0; ld: row pitch in elements (multiple of 8).
  // idx: optional row map (tile row -> global row), rows >= rows_valid are zero.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, const int32_t* idx,
                                       int row0, int rows_valid, int tid) {
    const int c = tid & 7;
    const int r = tid >> 3;
    ok = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = row0 + r + 32 * j;
      const bool v = row < rows_valid;
      int64_t g = 0;
      if (v) g = idx ? (int64_t)idx[row] : (int64_t)row;
      ptr[j] = reinterpret_cast<const uint4*>(base + g * ld) + c;
      ok |= (v ? 1u : 0u) << j;
    }
  }
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) reg[j] = ((ok >> j) & 1u) ? ptr[j][kt * 8] : zero4();
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
    const int c = tid & 7;
    const int r = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) lds[lds_slot(r + 32 * j, c)] = reg[j];
  }
};

// 8 x 8 transpose of bf16 elements held as 8 rows of 4 dwords.
// in[j] = row j (8 columns); out[c] = column c (8 rows, row 2e in the low half
// of dword e).
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4*j + d]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);              // o[4*c + e]
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = w[4 * (2 * e) + c / 2];
      const uint32_t b = w[4 * (2 * e + 1) + c / 2];
      // even column: low halves of a and b; odd column: high halves.
      o[4 * c + e] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u))
                             : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

// MN-major operand: element (k, col) at base[k * ld + col]; the tile covers
// columns col0 .. col0 + 255. Thread t loads rows kg*8 .. kg*8+7 (kg = t / 32)
// of the 64-row stage at columns (t % 32) * 8 .. + 7.
struct MNMajorStager {
  const uint16_t* p0;
  int64_t ld;
  int krow0;   // first k of this thread in a stage
  int k_valid; // k >= k_valid reads as zero
  bool col_ok;
  uint4 reg[8];

  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld_, int k_valid_, int col0,
                                       int cols_valid, int tid) {
    const int g = tid & 31;
    const int kg = tid >> 5;
    const int col = col0 + g * 8;
    col_ok = col + 8 <= cols_valid;
    ld = ld_;
    krow0 = kg * 8;
    k_valid = k_valid_;
    p0 = base + (int64_t)krow0 * ld + (col_ok ? col : 0);
  }
  __device__ __forceinline__ void load(int kt) {
    const uint16_t* p = p0 + (int64_t)kt * kBK * ld;
    const int k = kt * kBK + krow0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool v = col_ok && (k + j < k_valid);
      reg[j] = v ? *reinterpret_cast<const uint4*>(p + (int64_t)j * ld) : zero4();
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
    const int g = tid & 31;
    const int kg = tid >> 5;
    uint4 t[8];
    transpose8x8(reg, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) lds[lds_slot(g * 8 + c, kg)] = t[c];
  }
};

// ---------------------------------------------------------------------------
// Tile scheduling: persistent workgroups, XCD-aware grouped order.
// ---------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (chiplets), so block b
// runs on XCD b % 8. Slot s of round `it` is remapped so that the blocks of one
// XCD take consecutive logical tiles; logical tiles are ordered in groups of
// kGroupM m-tiles by all n-tiles (n fastest inside a column of the group), so
// the 32 concurrent tiles of an XCD form a 4 x 8 block that shares A and B
// panels in that XCD's L2.
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
// Main loop: accumulates one 256 x 256 tile into acc (wave's 4 x 4 blocks).
// lds_a / lds_b: [2][kStageChunks] uint4 each.
// ---------------------------------------------------------------------------

template <class SA, class SB>
__device__ __forceinline__ void mainloop(SA& sa, SB& sb, int nk, uint4* lds_a, uint4* lds_b,
                                         f32x16_t (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // wave row (m) 0..1
  const int wn = wave & 1;   // wave col (n) 0..1

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk <= 0) return;

  // Row of this lane inside each 32-row fragment block, and its k half.
  const int frow = lane & 31;
  const int khalf = lane >> 5;

  sa.load(0);
  sb.load(0);
  sa.store(lds_a, tid);
  sb.store(lds_b, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(kt + 1);
      sb.load(kt + 1);
    }
    const uint4* la = lds_a + cur * kStageChunks;
    const uint4* lb = lds_b + cur * kStageChunks;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + khalf;
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = la[lds_slot(wm * 128 + i * 32 + frow, chunk)];
        fa[i] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = lb[lds_slot(wn * 128 + j * 32 + frow, chunk)];
        fb[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      sa.store(lds_a + (cur ^ 1) * kStageChunks, tid);
      sb.store(lds_b + (cur ^ 1) * kStageChunks, tid);
    }
    __syncthreads();
  }
}

// Row (within the wave's 128-row half) held by accumulator register r of block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace lmh
