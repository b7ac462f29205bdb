// lmhead.hip - fused LM-head log-prob / entropy op for MI355X (gfx950):
// kernels and the C ABI declared in include/lmhead.h.
//
// Forward (prime-rl PR #3326 Overview: compact -> chunked log-prob/entropy ->
// expand back; SkyRL PR #2374 "How it works": one projection gives both the
// selected-token log-prob and the entropy):
//   1. k_compact_*   keep mask -> ascending kept rows, row -> compact position,
//                    target of each compact row (count, scan, write)
//   2. k_gather_cols X_c^T = X[kept]^T [h][c], the token operand of the logit
//                    GEMM (k = h rows, tokens contiguous)
//   3. k_fwd_tiles   Z^T tile = W[vtile] X[kept]^T on MFMA, never stored; per
//                    token: max, sum 2^(y), sum 2^(y) y over the tile's 256
//                    vocab rows (y = z log2 e - max), and the target logit
//   4. k_merge       fixed-order merge of the vocab-tile partials ->
//                    log-sum-exp, entropy, log-prob; scatter to kept rows
//   5. k_zero_skipped  +0.0 log-prob / entropy at skipped rows
// Backward (twinkle PR #283 section 1: recompute the softmax from saved inputs;
// SkyRL PR #2374 review: entropy is saved by the forward, not recomputed):
//   0. k_bwd_check   the saved state against the call's arguments (a
//                    mismatch leaves the saved state unread and dX, dW zero)
//   1. k_bwd_rows    per kept row: LSE, upstream grads and target folded into
//                    the coefficients of dz as a function of the logit
//   2. k_zero_rows   +0.0 dX rows at skipped positions
//   3. k_gather_cols X_c^T
//   4. per chunk of kept rows:
//      k_dz_tiles    recompute Z^T tile, p = exp(z - LSE),
//                    dZ = g_lp (onehot - p) - g_H p (z - LSE + H), bf16,
//                    stored token-major [c][v]
//      k_dx_tiles    dX[kept rows] = dZ W      (K = vocab); the tiles of a
//                    ragged last round as vocabulary pieces, summed in a
//                    fixed order by k_dx_reduce
//      k_dw_tiles    dW^T (+)= X_c^T dZ        (K = chunk rows), stored as dW
// Every GEMM reads a K-major A (W, dZ, X_c^T) and an MN-major B (X_c^T, W, dZ)
// as they are stored.
// Vocabulary-shard form (tensor parallelism over the weight rows; SkyRL PR
// #2374 gemini-code-assist and cursor reviews): the same kernels on a slice
// of the weight rows. Compaction and k_bwd_rows subtract the slice's first
// row from the targets, the tile merge writes per-row statistics records
// instead of log-probs (k_merge<true>), and k_merge_shards combines the
// records of all slices into the whole op's outputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/lmhead.h"
#include "gemm_core.h"
#include "launch.h"

#define LMH_API extern "C" __attribute__((visibility("default")))

namespace lmh {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Default token chunk: the largest multiple of 256 rows whose bf16 dZ buffer
// fits this budget. The pages' fused head defaults to 8192 rows to bound
// memory on an 80 GB part; with 288 GB of HBM the budget admits a whole
// 16K-token batch at V = 131072 (4 GiB of dZ), which saves the
// read-modify-write of dW between chunks.
constexpr int64_t kDefaultDzBudget = int64_t(8) << 30;
constexpr int kVersion = 300;  // 0.3.0: block-sparse forward, MFMA ceiling probe

// ---------------------------------------------------------------------------
// Saved-state layout (device memory, filled by the forward).
// ---------------------------------------------------------------------------
struct SavedHeader {
  int32_t n_kept;
  int32_t status;      // lmhead_status of the forward's device-side checks
  int32_t N, H, V;     // of the forward call (V: the whole vocabulary)
  int32_t flags;       // kFlag* below
  int32_t bwd_status;  // lmhead_status of the last backward's consistency check
};
constexpr int kFlagReturnEntropy = 1;
constexpr int kFlagEntropyGrad = 2;
constexpr int kFlagBlockSparse = 4;
constexpr int kFlagComplete = 8;  // LSE and entropy of every kept row are written
constexpr size_t kHeaderBytes = 1024;

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct SavedView {
  SavedHeader* hdr;
  int32_t* kept_idx;  // [N] ascending kept rows (first n_kept valid)
  int32_t* pos;       // [N] compact position of each row, -1 if skipped
  float* lse;         // [N] log-sum-exp per kept row (compact order)
  float* ent;         // [N] entropy per kept row (compact order)
};

static inline size_t saved_bytes_for(int64_t N) {
  return kHeaderBytes + 4 * align256((size_t)N * 4);
}

static inline SavedView saved_view(void* base, int64_t N) {
  char* p = static_cast<char*>(base);
  const size_t a = align256((size_t)N * 4);
  SavedView v;
  v.hdr = reinterpret_cast<SavedHeader*>(p);
  v.kept_idx = reinterpret_cast<int32_t*>(p + kHeaderBytes);
  v.pos = reinterpret_cast<int32_t*>(p + kHeaderBytes + a);
  v.lse = reinterpret_cast<float*>(p + kHeaderBytes + 2 * a);
  v.ent = reinterpret_cast<float*>(p + kHeaderBytes + 3 * a);
  return v;
}

static inline int n_vtiles(int64_t V) { return (int)((V + kBM - 1) / kBM); }

// The stage shift for nk stages: the rotation runs pairs of stages, so an
// odd count gets one padding stage.
__host__ __device__ constexpr int shift_for(int nk) { return stage_shift(nk + (nk & 1)); }
static __host__ __device__ constexpr int64_t round_up(int64_t x, int64_t m) {
  return (x + m - 1) / m * m;
}

// Row padding of the backward's own buffers, dZ and the chunk's X_c^T: 64
// elements (128 bytes). Their natural pitches are powers of two at the usual
// shapes (V = 131072 gives dZ rows of 256 KiB, C = 16384 rows of X_c^T of
// 32 KiB), which map the 32 k rows a GEMM stage loads from them, and the
// same rows of the other tiles of an XCD, to few L2 sets. Measured at N 16384,
// H 4096, V 131072: dW's L2 refills 52.5 -> 29.7 GB per launch, its time
// 11.9 -> 11.6 ms (128 and 256 elements of padding were no better).
constexpr int64_t kPitchPad = 64;

// Size limits. Every GEMM operand is addressed through per-wave buffer
// descriptors whose record counts and offsets must stay below 2^31 bytes:
// a K-major operand's row pitch below kMaxALd elements, an MN-major one's
// below kMaxBLd (gemm_core.h). The operands and their pitches:
//   W [V][H]            pitch H                      (A of the logit GEMMs, B of dX)
//   X_c^T, forward      pitch N rounded to 64        (B of the logit GEMM)
//   X_c^T, backward     pitch C + 64, C the chunk    (B of dZ, A of dW)
//   dZ [C][ldz]         pitch V rounded to 256, + 64 (A of dX, B of dW)
// so H <= 2^20, V <= 2^22, N <= 2^24 and C <= 2^22 keep every pitch inside
// its bound, and every tile count inside int32: (V / 256) (N / 256) <= 2^30.
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxH = int64_t(1) << 20;
constexpr int64_t kMaxV = int64_t(1) << 22;
constexpr int64_t kMaxChunk = int64_t(1) << 22;
static_assert(kMaxH < kMaxALd && round_up(kMaxV, 256) + kPitchPad < kMaxALd &&
                  kMaxChunk + kPitchPad < kMaxALd,
              "K-major operand pitches");
static_assert(round_up(kMaxN, 64) < kMaxBLd && kMaxH < kMaxBLd && kMaxChunk + kPitchPad < kMaxBLd,
              "MN-major operand pitches");
static_assert((kMaxV / 256) * (kMaxN / 256) < (int64_t(1) << 31), "tile indices");

// Pitch of the transposed kept rows X_c^T [H][ldc].
static inline int64_t ldc_of(int64_t N) { return round_up(N, 64); }

// Rows of the per-token arrays the GEMM epilogues read: whole 256-token tiles.
static inline int64_t tile_rows(int64_t N) { return round_up(N, 256); }

// Forward workspace: tile-queue counters | compact targets [tile_rows] |
// target logits [N] (first the compaction's per-chunk counts and flags) |
// partial m, s, b [n_vt][N] each | X_c^T [H][ldc] (bf16).
struct FwdWs {
  size_t q, tg, zt, pm, ps, pb, xct, total;
};
constexpr int kQueueInts = 8;  // one tile-queue counter per XCD
static inline FwdWs fwd_ws(int64_t N, int64_t H, int64_t V) {
  const size_t nv = (size_t)n_vtiles(V);
  FwdWs w;
  w.q = 0;
  w.tg = w.q + align256(kQueueInts * 4);
  w.zt = w.tg + align256((size_t)tile_rows(N) * 4);
  w.pm = w.zt + align256((size_t)N * 4);
  w.ps = w.pm + align256(nv * (size_t)N * 4);
  w.pb = w.ps + align256(nv * (size_t)N * 4);
  w.xct = w.pb + align256(nv * (size_t)N * 4);
  w.total = w.xct + align256((size_t)H * (size_t)ldc_of(N) * 2);
  return w;
}

// Backward geometry: chunk capacity C (rows, multiple of 256), the pitch ldc
// of the chunk's X_c^T (C + kPitchPad) and the dZ pitch ldz (V rounded up to
// 256, + kPitchPad).
struct BwdGeom {
  int64_t C, ldc, ldz;
};
static inline BwdGeom bwd_geom(int64_t N, int64_t V, int64_t token_chunk) {
  BwdGeom g;
  int64_t want = token_chunk;
  g.ldz = round_up(V, 256) + kPitchPad;
  if (want <= 0) {
    want = kDefaultDzBudget / (2 * g.ldz) / 256 * 256;
    if (want < 256) want = 256;
  }
  want = std::min(want, kMaxChunk);  // a memory knob: results do not depend on it
  g.C = N > 0 ? std::min(round_up(want, 256), round_up(N, 256)) : 0;
  g.ldc = g.C + kPitchPad;
  return g;
}

// dX tail split. The dX GEMM of a chunk has ceil(rows / 256) x ceil(H / 256)
// tiles of K = V, each a long run (2.8 ms at V = 131072). When the tiles past
// the last whole round of the grid -- the tail -- number at most
// 256 (S - 1) / S, each tail tile is cut into S pieces of the K range, which
// the whole chip runs, and a fixed-order sum of the pieces writes the tile:
// 672 tiles on 256 CUs take 2.625 tile times instead of 3, and the 2 tiles of
// a 128-row batch at H 512 run as 16 pieces instead of on 2 CUs. Only for
// V >= kDxSplitMinV: a piece then has at least 256 vocabulary rows (8 stages),
// enough to pay for its prologue, epilogue and share of the sum (a piece
// costs about 12 us of fixed work, a whole tile 0.66 us per 32 vocabulary
// rows). Pieces are kp = a multiple of 64 vocabulary rows, with S kp within
// the dZ row pitch (V rounded up to 256) so that no piece reads past its
// row: S = 8 where that holds, else 4 (the pitch is a multiple of 4 x 64).
constexpr int64_t kDxSplitMinV = 2048;
static inline int64_t dz_pitch(int64_t V) { return round_up(V, 256); }
static inline int dx_piece_k_for(int64_t V, int S) { return (int)round_up((V + S - 1) / S, 64); }
static inline int dx_pieces(int64_t V) {
  if (V < kDxSplitMinV) return 1;
  return 8 * (int64_t)dx_piece_k_for(V, 8) <= dz_pitch(V) ? 8 : 4;
}
static inline int dx_piece_k(int64_t V) { return dx_piece_k_for(V, dx_pieces(V)); }
static inline int64_t dx_tiles_per_chunk(int64_t C, int64_t H) {
  return (C / kBM) * ((H + kBN - 1) / kBN);
}
static inline int dx_tail_max(int64_t C, int64_t H, int64_t V) {
  const int S = dx_pieces(V);
  if (S == 1) return 0;
  return (int)std::min<int64_t>(256 * (S - 1) / S, dx_tiles_per_chunk(C, H));
}

// Backward workspace: the checked copy of the saved header | tile-queue
// counters (four launches per chunk) | per-row dZ coefficients (float4) and
// compact targets [tile_rows] | X_c^T of one chunk [H][ldc] | dZ [C][ldz], both
// bf16 | fp32 partial dX tiles of a split tail [tail max x pieces][256][256].
constexpr int kBwdQueueSets = 4;  // dz, dx, dx pieces, dw
struct BwdWs {
  size_t chk, q, rc, tg, xct, dz, part, total;
  int64_t nq;  // counters
};
static inline BwdWs bwd_ws(int64_t N, int64_t H, int64_t V, int64_t token_chunk) {
  const BwdGeom g = bwd_geom(N, V, token_chunk);
  BwdWs w;
  const int64_t nchunks = N > 0 ? (N + g.C - 1) / g.C : 1;
  w.nq = nchunks * kBwdQueueSets * kQueueInts;
  w.chk = 0;
  w.q = w.chk + align256(sizeof(SavedHeader));
  w.rc = w.q + align256((size_t)w.nq * 4);
  w.tg = w.rc + align256((size_t)tile_rows(N) * 16);
  w.xct = w.tg + align256((size_t)tile_rows(N) * 4);
  w.dz = w.xct + align256((size_t)H * (size_t)g.ldc * 2);
  w.part = w.dz + align256((size_t)g.C * (size_t)g.ldz * 2);
  w.total = w.part + (size_t)dx_tail_max(g.C, H, V) * dx_pieces(V) * kBM * kBN * 4;
  return w;
}

// ---------------------------------------------------------------------------
// Compaction, in three launches so that it scales with N: every workgroup owns
// kCompactRows consecutive rows (16 per thread), (1) counts the rows it lists
// and flags kept rows whose target is out of range, (2) one workgroup scans
// the per-chunk counts into offsets and writes the saved header, (3) every
// workgroup writes its rows at its offset. The per-chunk counts and flags live
// in the forward's target-logit array, which the projection fills only later.
//
// Rows are taken in blocks of `block` consecutive rows: a block is listed,
// whole, when any of its rows is kept. block = 1 lists exactly the kept rows
// (the compacting forward); block = 256 lists every row of each 256-row tile
// that holds a kept row, in place, so that the GEMMs skip only the tiles whose
// rows are all masked (the block-sparse forward). A listed row that is not
// kept gets pos = -2 - c (c its listed position) and target -1; the merge
// and the backward give it +0.0 outputs and an all-zero dz row.
// ---------------------------------------------------------------------------
constexpr int kCompactThreads = 256;
constexpr int kCompactPerThread = 16;
constexpr int kCompactRows = kCompactThreads * kCompactPerThread;  // 4096, a whole number of 256-row blocks
constexpr int kScanThreads = 1024;

static inline int compact_chunks(int64_t N) { return (int)((N + kCompactRows - 1) / kCompactRows); }

// Kept-row bits of this thread's 16 rows starting at r0 (bit j: row r0 + j),
// and whether each row is listed: with block = 256 the 16 threads of a block
// (16 adjacent lanes) combine their bits.
__device__ __forceinline__ void compact_bits(const uint8_t* __restrict__ keep, int N, int r0,
                                             int block, uint32_t& kept, uint32_t& listed) {
  kept = 0;
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kCompactPerThread; ++j) {
    const int i = r0 + j;
    if (i < N) {
      valid |= 1u << j;
      if (keep == nullptr || keep[i] != 0) kept |= 1u << j;
    }
  }
  listed = kept;
  if (block > 1) {
    int any = kept != 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) any |= __shfl_xor(any, d, 16);
    listed = any ? valid : 0u;
  }
}

// Exclusive prefix sum over a workgroup of kCompactThreads threads.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kCompactThreads; off <<= 1) {
    const int u = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += u;
    __syncthreads();
  }
  const int incl = sh[tid];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kCompactThreads) void k_compact_count(
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ targets, int N, int V,
    int block, int* __restrict__ scratch, int nchunks) {
  __shared__ int sh[kCompactThreads];
  const int r0 = blockIdx.x * kCompactRows + threadIdx.x * kCompactPerThread;
  uint32_t kept, listed;
  compact_bits(keep, N, r0, block, kept, listed);
  int bad = 0;
  for (uint32_t k = kept; k; k &= k - 1) {
    const int t = targets[r0 + __builtin_ctz(k)];
    bad |= (t < 0 || t >= V);
  }
  const int cnt = __builtin_popcount(listed);
  const int before = wg_exclusive_scan(cnt, sh);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == kCompactThreads - 1) {
    scratch[blockIdx.x] = before + cnt;
    scratch[nchunks + blockIdx.x] = bad;
  }
}

// One workgroup: per-chunk counts -> exclusive offsets (in place), and the
// saved header.
__global__ __launch_bounds__(kScanThreads) void k_compact_scan(int* __restrict__ scratch,
                                                               int nchunks, int N, int H, int V,
                                                               int flags,
                                                               SavedHeader* __restrict__ hdr) {
  __shared__ int sh[kScanThreads];
  const int tid = threadIdx.x;
  const int seg = (nchunks + kScanThreads - 1) / kScanThreads;
  const int beg = min(nchunks, tid * seg), end = min(nchunks, beg + seg);
  int sum = 0, bad = 0;
  for (int b = beg; b < end; ++b) {
    sum += scratch[b];
    bad |= scratch[nchunks + b];
  }
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int u = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += u;
    __syncthreads();
  }
  int o = sh[tid] - sum;
  for (int b = beg; b < end; ++b) {
    const int c = scratch[b];
    scratch[b] = o;
    o += c;
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    hdr->n_kept = sh[kScanThreads - 1];
    hdr->status = bad ? LMHEAD_ERR_TARGET_RANGE : LMHEAD_OK;
    hdr->N = N;
    hdr->H = H;
    hdr->V = V;
    hdr->flags = flags;
    hdr->bwd_status = LMHEAD_OK;
  }
}

__global__ __launch_bounds__(kCompactThreads) void k_compact_write(
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ targets, int N, int block,
    const int* __restrict__ scratch, const SavedHeader* __restrict__ hdr,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ pos, int32_t* __restrict__ tg,
    int tg_rows, int vocab_start) {
  __shared__ int sh[kCompactThreads];
  const int r0 = blockIdx.x * kCompactRows + threadIdx.x * kCompactPerThread;
  uint32_t kept, listed;
  compact_bits(keep, N, r0, block, kept, listed);
  int o = scratch[blockIdx.x] + wg_exclusive_scan(__builtin_popcount(listed), sh);
#pragma unroll
  for (int j = 0; j < kCompactPerThread; ++j) {
    const int i = r0 + j;
    if (i >= N) break;
    if (!((listed >> j) & 1u)) {
      pos[i] = -1;
      continue;
    }
    kept_idx[o] = i;
    if ((kept >> j) & 1u) {
      pos[i] = o;
      tg[o] = targets[i] - vocab_start;  // row of the weight this call reads
    } else {
      pos[i] = -2 - o;
      tg[o] = -1;
    }
    ++o;
  }
  // compact targets past the listed rows: -1 matches no vocabulary row; this
  // workgroup fills its share of [n_kept, tg_rows)
  const int total = hdr->n_kept;
  const int c0 = total + blockIdx.x * kCompactRows;
  for (int c = c0 + threadIdx.x; c < min(tg_rows, c0 + kCompactRows); c += kCompactThreads)
    tg[c] = -1;
}

// ---------------------------------------------------------------------------
// Online softmax statistics in base-2 units.
// A partial (m, s, b) over a set S of logits z means, with y = z log2(e):
//   m = max_S y,  s = sum_S 2^(y - m),  b = sum_S 2^(y - m) (y - m).
// Two partials merge exactly (up to rounding) as
//   m = max(m1, m2), a_k = 2^(m_k - m), s = sum a_k s_k,
//   b = sum a_k (b_k + (m_k - m) s_k).
// Then LSE = (m + log2 s) ln 2 and entropy = (log2 s - b / s) ln 2. The
// scale factors use the hardware exp2: m_k - m <= 0, and a partial more than
// 126 (base-2 units) below the maximum contributes below 2^-126 of it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stat_merge(float& m, float& s, float& b, float m2, float s2,
                                           float b2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  float a1 = 0.f, a2 = 0.f, t1 = 0.f, t2 = 0.f;
  if (m != -INFINITY) {
    const float d = m - mn;
    a1 = __builtin_amdgcn_exp2f(d);
    t1 = a1 * (b + d * s);
    a1 *= s;
  }
  if (m2 != -INFINITY) {
    const float d = m2 - mn;
    a2 = __builtin_amdgcn_exp2f(d);
    t2 = a2 * (b2 + d * s2);
    a2 *= s2;
  }
  m = mn;
  s = a1 + a2;
  b = t1 + t2;
}

// ---------------------------------------------------------------------------
// Per-tile phase clocks of the four tile kernels, compiled in only with
// LMHEAD_TILE_CLOCKS (an instrumented build for measurement; the default
// build contains none of it). Each workgroup reads the shader clock
// (s_memtime) and the constant 100 MHz clock (s_memrealtime) when it has
// taken a tile, after the tile's main loop and after its epilogue, and
// thread 0 adds the totals into per-kernel device counters when the
// workgroup exits: main-loop and epilogue time and cycles, time spent taking
// tiles, and the tile count. lmhead_tile_clocks (same build only) reads them.
// Per XCD it also keeps the earliest workgroup start and the latest
// workgroup exit of each kernel (lmhead_tile_clocks_xcd), which show how far
// apart the XCDs finish a launch.
// ---------------------------------------------------------------------------
enum { kClkFwd = 0, kClkDz = 1, kClkDx = 2, kClkDw = 3 };
#ifdef LMHEAD_TILE_CLOCKS
__device__ unsigned long long g_tile_clock[4][8];
__device__ unsigned long long g_xcd_clock[4][kXcds][2];  // earliest start, latest exit
struct TileClock {
  uint64_t r0, r_end, r_a = 0, r_b = 0, c_a = 0, c_b = 0;
  uint64_t main = 0, epi = 0, next = 0, n = 0, cmain = 0, cepi = 0;
  __device__ TileClock() : r0(__builtin_amdgcn_s_memrealtime()), r_end(r0) {}
  __device__ void tile_start() {
    r_a = __builtin_amdgcn_s_memrealtime();
    c_a = __builtin_amdgcn_s_memtime();
    next += r_a - r_end;
  }
  __device__ void main_done() {
    r_b = __builtin_amdgcn_s_memrealtime();
    c_b = __builtin_amdgcn_s_memtime();
    main += r_b - r_a;
    cmain += c_b - c_a;
  }
  __device__ void tile_done() {
    r_end = __builtin_amdgcn_s_memrealtime();
    epi += r_end - r_b;
    cepi += __builtin_amdgcn_s_memtime() - c_b;
    ++n;
  }
  __device__ void flush(int k) {
    if (threadIdx.x != 0) return;
    const unsigned long long v[7] = {main, epi, next, n, cmain, cepi, 1};
    for (int i = 0; i < 7; ++i) atomicAdd(&g_tile_clock[k][i], v[i]);
    const int x = xcd_id();
    atomicMin(&g_xcd_clock[k][x][0], (unsigned long long)r0);
    atomicMax(&g_xcd_clock[k][x][1], (unsigned long long)__builtin_amdgcn_s_memrealtime());
  }
};
#else
struct TileClock {
  __device__ void tile_start() {}
  __device__ void main_done() {}
  __device__ void tile_done() {}
  __device__ void flush(int) {}
};
#endif

// ---------------------------------------------------------------------------
// Gathered transpose of the kept rows through LDS in 64 x 64 tiles (bf16),
// zero-filled past the kept rows so that every tile reads finite values:
//   k_gather_cols : XcT[h][c] = X[kept_idx[c0 + c]][h] for c < ld (zero where
//                   c0 + c >= n_kept); the forward gathers every kept row
//                   (c0 = 0), the backward one chunk of them at a time
// ---------------------------------------------------------------------------
constexpr int kTp = 64;
constexpr int kTpPitch = kTp + 8;  // 144-byte rows

// LDS layout of the tile: element (r, c) sits in 8-element chunk
// (c / 8) ^ (r / 8) of row r. A thread of the transposed read below takes
// one column c at 8 rows r spaced 1 apart within one 8-row group g = r / 8,
// and the 8 lanes that share c read the groups g = 0..7; unswizzled, those
// groups lie 8 rows = 288 dwords apart, the same bank for every group, while
// the swizzle moves group g to chunk (c / 8) ^ g, 4 banks further per group.
__device__ __forceinline__ int tile_col(int r, int c) { return (((c >> 3) ^ (r >> 3)) << 3) | (c & 7); }

// Loads rows r (< 64) of the tile as 8-element chunks: src(r) is the row's
// first element, or null for a zero row.
template <class RowPtr>
__device__ __forceinline__ void tile_load(uint16_t (*t)[kTpPitch], RowPtr src) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = tid / 8 + 32 * it;
    const int ch = tid % 8;
    const uint16_t* p = src(r);
    const uint4 x = p ? *reinterpret_cast<const uint4*>(p + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&t[r][tile_col(r, ch * 8)]) = x;
  }
}

// Writes the transpose of the LDS tile: out row h (< 64) gets t[.][h].
__device__ __forceinline__ void tile_store_t(uint16_t (*t)[kTpPitch], uint16_t* __restrict__ out,
                                             int64_t ld_out) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int h = tid / 8 + 32 * it;
    const int ch = tid % 8;
    const int col = tile_col(ch * 8, h);  // rows ch * 8 .. ch * 8 + 7 share it
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[ch * 8 + 2 * e][col] | ((uint32_t)t[ch * 8 + 2 * e + 1][col] << 16);
    *reinterpret_cast<uint4*>(out + (int64_t)h * ld_out + ch * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(256) void k_gather_cols(const uint16_t* __restrict__ X,
                                                     const SavedHeader* __restrict__ hdr,
                                                     const int32_t* __restrict__ kept_idx,
                                                     int first, int H,
                                                     uint16_t* __restrict__ XcT, int64_t ldc) {
  __shared__ uint16_t t[kTp][kTpPitch];
  const int n_kept = hdr->n_kept;
  const int c0 = blockIdx.x * kTp, h0 = blockIdx.y * kTp;
  tile_load(t, [&](int r) -> const uint16_t* {
    const int c = first + c0 + r;
    return c < n_kept ? X + (int64_t)kept_idx[c] * H + h0 : nullptr;
  });
  __syncthreads();
  tile_store_t(t, XcT + (int64_t)h0 * ldc + c0, ldc);
}

// ---------------------------------------------------------------------------
// Forward tiles: M = vocab (A = W rows), N = kept tokens (B = X_c^T), K = H.
// The epilogue reduces over the tile's 256 vocab rows per token.
// ---------------------------------------------------------------------------
struct FwdParams {
  const uint16_t* W;    // [V][H]
  const uint16_t* XcT;  // [H][ldc]
  const int32_t* tg;    // [tile_rows] target of each compact row, -1 past the kept rows
  const SavedHeader* hdr;
  int H, V, n_vt;
  int64_t ldc;
  int64_t ldp;  // pitch (elements) between vocab tiles in the partial arrays
  float* pm;
  float* ps;
  float* pb;
  float* zt;
  int* queue;  // tile-queue counters of this launch (zero before it)
  int steal;
};

template <int SHIFT>
__global__ __launch_bounds__(kThreads, 1) void k_fwd_tiles(FwdParams P) {
  LMH_DECLARE_RING;
  // per-token partials of the two wave rows x four lane groups; reuses ring
  // slot 0 after the main loop (rows padded to 272 floats: the four lane
  // groups of a write then fall in different banks)
  constexpr int kRedPitch = kBN + 16;
  static_assert(8 * 3 * kRedPitch * 4 <= kASlotBytes, "the partials fit one A slot");
  float (*red)[3][kRedPitch] = reinterpret_cast<float (*)[3][kRedPitch]>(ra0);

  const int rows = P.hdr->n_kept;
  const int mt = P.n_vt;
  const int nt = (rows + kBN - 1) / kBN;
  const int ntiles = mt * nt;
  const int tid = threadIdx.x;
  const int nk = P.H / kBK;

  TileQueue q(P.queue, ntiles, P.steal);
  TileClock clk;
  for (;;) {
    const int t = q.next(ring.b[bcast_slot<SHIFT>()]);
    if (t < 0) break;
    clk.tile_start();
    int tm, tn;
    tile_coords<LMH_GM_FWD>(t, mt, nt, tm, tn);

    // targets of this lane's eight tokens (columns 16 j + lane % 16 of the
    // wave's 128), loaded before the main loop so that their latency is
    // hidden under it
    int tgt[8];
    {
      const int* tp = P.tg + tn * kBN + (wave_fresh() & 1) * 128 + (lane_fresh() & 15);
#pragma unroll
      for (int j = 0; j < 8; ++j) tgt[j] = tp[j * 16];
    }

    ASrc A;
    BSrc B;
    A.init(P.W + (int64_t)tm * kBM * P.H, P.H, P.V - tm * kBM);
    B.init(P.XcT + (int64_t)tn * kBN, P.ldc, P.H, rows - tn * kBN);
    Acc acc;
    mainloop<SHIFT>(A, B, nk, ring, acc);
    clk.main_done();
    q.claim_ahead();
    // per-tile lane values (see lane_fresh): nothing lane-derived is hoisted
    // out of the tile loop to be spilled across the main loop
    const int lane = lane_fresh(), wave = wave_fresh();
    const int wm = wave >> 1, wn = wave & 1;

    const int vbase = tm * kBM + wm * 128;
    const bool full = vbase + 128 <= P.V;
    const int vlim = P.V - vbase - acc_row_lane(lane);  // rows acc_row_fixed < vlim are valid
    lds_barrier();  // every wave is done reading the ring
    const int fence = acc_read_fence();
    // Per token (column 16 j + lane % 16 of the wave): m = max y,
    // s = sum 2^(y - m) and b = sum 2^(y - m) (y - m) over this lane's 32
    // vocabulary rows (16 i + 4 (lane / 16) + r), staged in LDS with the
    // token's seven other partials (the three other lanes of the wave that
    // hold its rows, and the other wave row) for one merge per token; then
    // the target pick. The masked form leaves out rows at or past V, which
    // only the last vocabulary tile has; a lane with no valid row gives the
    // empty partial (-inf, 0, 0).
    auto columns = [&](auto masked_t) {
      constexpr bool kMasked = decltype(masked_t)::value;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cl = wn * 128 + j * 16 + (lane & 15);  // token inside the tile
        const int c = tn * kBN + cl;                     // compact row
        // this lane's 32 logits of the token, each accumulator read once; the
        // masked form replaces rows at or past V by a large finite negative
        // logit, whose 2^(y - m) is exactly 0 next to any real maximum while
        // 0 * y stays finite
        // (the row limit is made opaque per column so that the 32 row masks
        // are recomputed, not kept in scalar registers across columns)
        int vl = vlim;
        if (kMasked) asm volatile("" : "+v"(vl));
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[i * 4 + r] =
                (!kMasked || acc_row_fixed(i, r) < vl) ? acc_read(acc[i][j][r], fence) : -1e30f;
        float mx = v[0];
#pragma unroll
        for (int k = 1; k < 32; ++k) mx = fmaxf(mx, v[k]);
        if (kMasked && vlim <= 0) mx = -INFINITY;  // no valid row: the empty partial
        float m = (mx == -INFINITY) ? -INFINITY : mx * kLog2e;
        float s = 0.f, b = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            // y = z log2 e - m: 0 up to the rounding of m at the maximum
            const float y = fmaf(v[k], kLog2e, -m);
            const float e = __builtin_amdgcn_exp2f(y);
            s += e;
            b = fmaf(e, y, b);
          }
        }
        {
          const int pset = wm * 4 + (lane >> 4);  // wave row, lane group
          red[pset][0][cl] = m;
          red[pset][1][cl] = s;
          red[pset][2][cl] = b;
        }
        // exactly one lane in the grid holds z[t] for a kept token (the
        // target of a token past the kept rows is -1 and never hits): row
        // local = 16 i + 4 g + r of the wave's 128 sits in lane group g
        const int local = tgt[j] - vbase;
        const bool hit = local >= 0 && local < 128 && ((local >> 2) & 3) == (lane >> 4);
        if (hit) {
          const int want = (local >> 4) * 4 + (local & 3);
          float z = 0.f;
#pragma unroll
          for (int k = 0; k < 32; ++k) z = (want == k) ? v[k] : z;
          P.zt[c] = z;
        }
        // one column at a time: keeps the copies of the accumulators out of
        // the way of the other columns (no spills)
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (full)
      columns(std::false_type{});
    else
      columns(std::true_type{});
    lds_barrier();  // every lane has staged its partials
    {
      const int cl = tid;  // one token per thread
      const int c = tn * kBN + cl;
      // the token's eight partials in a fixed order: their maximum first,
      // then the sums rescaled to it; an empty partial adds nothing
      float pm8[8], ps8[8], pb8[8];
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pm8[k] = red[k][0][cl];
        ps8[k] = red[k][1][cl];
        pb8[k] = red[k][2][cl];
        m = fmaxf(m, pm8[k]);
      }
      float s = 0.f, b = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (pm8[k] != -INFINITY) {
            const float d = pm8[k] - m;
            const float a = __builtin_amdgcn_exp2f(d);
            s = fmaf(a, ps8[k], s);
            b = fmaf(a, fmaf(d, ps8[k], pb8[k]), b);
          }
        }
      }
      if (c < rows) {
        const int64_t o = (int64_t)tm * P.ldp + c;
        P.pm[o] = m;
        P.ps[o] = s;
        P.pb[o] = b;
      }
    }
    clk.tile_done();
  }
  clk.flush(kClkFwd);
}

// ---------------------------------------------------------------------------
// Merge of the vocab-tile partials, in ascending tile order within each of 8
// interleaved splits, then splits 0..7 in order (32 rows per workgroup, so a
// split reads 128 contiguous bytes of each partial array per tile). The full op writes the saved
// LSE and entropy and scatters log-prob / entropy to the kept rows. The
// vocabulary-shard form (kRecord) writes each kept row's statistics over the
// shard instead, in natural-log units: {m, s, b, z_t} with m = max z,
// s = sum e^(z - m), b = sum e^(z - m) (z - m), and z_t the target logit if
// the target lies in the shard, else NaN.
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 32;
constexpr int kMergeSplits = 256 / kMergeRows;

template <bool kRecord>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ pm,
                                               const float* __restrict__ ps,
                                               const float* __restrict__ pb,
                                               const float* __restrict__ zt, int64_t ldp, int n_vt,
                                               const int32_t* __restrict__ tg, int V,
                                               SavedView sv, float* __restrict__ logp,
                                               float* __restrict__ entropy,
                                               float4* __restrict__ rec) {
  __shared__ float sh[3][kMergeSplits][kMergeRows];
  const int rows = sv.hdr->n_kept;
  const int r = threadIdx.x & (kMergeRows - 1);
  const int split = threadIdx.x / kMergeRows;
  const int c = blockIdx.x * kMergeRows + r;
  if (blockIdx.x * kMergeRows >= rows) return;
  float m = -INFINITY, s = 0.f, b = 0.f;
  if (c < rows) {
#pragma unroll 4
    for (int vt = split; vt < n_vt; vt += kMergeSplits) {
      const int64_t o = (int64_t)vt * ldp + c;
      stat_merge(m, s, b, pm[o], ps[o], pb[o]);
    }
  }
  sh[0][split][r] = m;
  sh[1][split][r] = s;
  sh[2][split][r] = b;
  __syncthreads();
  if (split == 0 && c < rows) {
    for (int k = 1; k < kMergeSplits; ++k) stat_merge(m, s, b, sh[0][k][r], sh[1][k][r], sh[2][k][r]);
    const int row = sv.kept_idx[c];
    const int t = tg[c];
    const bool has_t = t >= 0 && t < V;
    if constexpr (kRecord) {
      rec[row] = make_float4(m * kLn2, s, b * kLn2, has_t ? zt[c] : __builtin_nanf(""));
    } else {
      const bool live = sv.pos[row] == c;  // a listed row of a masked block is not kept
      const float l2s = log2f(s);
      const float lse = (m + l2s) * kLn2;
      const float ent = (l2s - b / s) * kLn2;
      const float lp = has_t ? zt[c] - lse : __builtin_nanf("");
      sv.lse[c] = lse;
      sv.ent[c] = ent;
      logp[row] = live ? lp : 0.f;
      if (entropy) entropy[row] = live ? ent : 0.f;
    }
  }
}

// Record of a skipped row in the vocabulary-shard form: the empty partial.
__global__ void k_skipped_records(const int32_t* __restrict__ pos, int N, float4* __restrict__ rec) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N && pos[i] < 0) rec[i] = make_float4(-INFINITY, 0.f, 0.f, __builtin_nanf(""));
}

// Combines the records of P vocabulary shards (disjoint ranges that together
// cover the vocabulary), in shard order, into the full op's outputs: the
// statistics merge as in stat_merge, and the target logit comes from the one
// shard that holds the target (NaN if none does). Writes the saved LSE and
// entropy of every kept row, log-prob / entropy of every row (+0.0 where
// skipped), and the flags into the saved header.
__global__ __launch_bounds__(256) void k_merge_shards(const float4* __restrict__ rec, int P,
                                                      int64_t N, SavedView sv, int flags,
                                                      float* __restrict__ logp,
                                                      float* __restrict__ entropy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) sv.hdr->flags = flags | kFlagComplete;
  if (i >= N) return;
  const int c = sv.pos[i];
  if (c < 0) {
    logp[i] = 0.f;
    if (entropy) entropy[i] = 0.f;
    return;
  }
  float m = -INFINITY, s = 0.f, b = 0.f, z = __builtin_nanf("");
  for (int p = 0; p < P; ++p) {
    const float4 q = rec[(int64_t)p * N + i];
    stat_merge(m, s, b, q.x * kLog2e, q.y, q.z * kLog2e);  // to base-2 units
    if (!(q.w != q.w) && z != z) z = q.w;
  }
  const float l2s = log2f(s);
  const float lse = (m + l2s) * kLn2;
  const float ent = (l2s - b / s) * kLn2;
  sv.lse[c] = lse;
  sv.ent[c] = ent;
  logp[i] = z - lse;
  if (entropy) entropy[i] = ent;
}

__global__ void k_zero_skipped(const int32_t* __restrict__ pos, int N, float* __restrict__ logp,
                               float* __restrict__ entropy) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N && pos[i] < 0) {
    logp[i] = 0.f;
    if (entropy) entropy[i] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Backward kernels.
// ---------------------------------------------------------------------------
// Zeroes n ints (the tile-queue counters of the launches that follow).
__global__ void k_zero_ints(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// The backward's check of the saved state against its own arguments (the
// saved header is on the device, and the library does not synchronise).
// `chk` receives a copy of the header whose n_kept every backward kernel
// reads: the saved count when the state belongs to this call, else 0, so a
// mismatched call computes nothing from the saved state, and k_zero_rows
// then clears every dX row (status != OK). The outcome is also written to the
// saved header's bwd_status, which lmhead_check_status reports. The state
// belongs to the call when N and H match, the vocabulary matches (the whole
// vocabulary, or for a vocabulary shard a range inside the forward's
// vocabulary), the forward completed LSE and entropy (a shard forward's
// state only after lmhead_merge_partials), and the entropy-gradient flag
// matches the forward's.
__global__ void k_bwd_check(SavedHeader* __restrict__ hdr, int N, int H, int V, int vocab_start,
                            int shard, int entropy_grad, SavedHeader* __restrict__ chk) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int flags = hdr->flags;
  const bool vocab_ok = shard ? (vocab_start >= 0 && (int64_t)vocab_start + V <= hdr->V)
                              : (hdr->V == V && vocab_start == 0);
  const bool ok = hdr->N == N && hdr->H == H && vocab_ok && (flags & kFlagComplete) &&
                  (((flags & kFlagEntropyGrad) != 0) == (entropy_grad != 0)) &&
                  hdr->n_kept >= 0 && hdr->n_kept <= N;
  SavedHeader c = *hdr;
  c.n_kept = ok ? hdr->n_kept : 0;
  c.status = ok ? LMHEAD_OK : LMHEAD_ERR_INVALID_ARG;
  *chk = c;
  hdr->bwd_status = c.status;
}

// +0.0 dX rows at skipped positions, or at every row when the saved state
// failed the backward's check. Workgroups stride over the rows (a launch may
// hold at most 2^32 work-items, fewer than one workgroup per row at N = 2^24).
constexpr int kZeroRowsGrid = 16384;
__global__ void k_zero_rows(const int32_t* __restrict__ pos, const SavedHeader* __restrict__ chk,
                            int N, int H, float* __restrict__ dX) {
  const bool all = chk->status != LMHEAD_OK;
  for (int i = blockIdx.x; i < N; i += gridDim.x) {
    if (!all && pos[i] >= 0) continue;
    float4* row = reinterpret_cast<float4*>(dX + (int64_t)i * H);
    for (int k = threadIdx.x; k < H / 4; k += blockDim.x) row[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Per compact row c, the coefficients of dz as a function of the logit z:
//   dz = p (ca + cb (z - LSE)) + g_lp [v = t],  p = 2^(z log2 e - LSE log2 e),
//   ca = -(g_lp + g_H H),  cb = -g_H,
// stored as {LSE log2 e, ca - cb LSE, cb, g_lp} with the target t beside it.
// Rows past the listed ones, and listed rows that are not kept (block-sparse
// forward), get zeros and target -1, so their dz is exactly 0.
__global__ __launch_bounds__(256) void k_bwd_rows(SavedView sv, const int32_t* __restrict__ targets,
                                                  const float* __restrict__ g_lp,
                                                  const float* __restrict__ g_h, int n_rows,
                                                  int vocab_start, float4* __restrict__ rc,
                                                  int32_t* __restrict__ tg) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n_rows) return;
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  int t = -1;
  const int row = c < sv.hdr->n_kept ? sv.kept_idx[c] : -1;
  if (row >= 0 && sv.pos[row] == c) {
    const float lse = sv.lse[c];
    const float glp = g_lp[row];
    const float gh = g_h ? g_h[row] : 0.f;
    const float ent = g_h ? sv.ent[c] : 0.f;
    const float ca = -(glp + gh * ent), cb = -gh;
    r = make_float4(lse * kLog2e, ca - cb * lse, cb, glp);
    t = targets[row] - vocab_start;  // row of the weight this call reads
  }
  rc[c] = r;
  tg[c] = t;
}

struct DzParams {
  const uint16_t* W;    // [V][H]
  const uint16_t* XcT;  // [H][ldc]: the chunk's kept rows, transposed
  const float4* rc;     // [tile_rows] dz coefficients per compact row (k_bwd_rows)
  const int32_t* tg;    // [tile_rows] target per compact row, -1 past the kept rows
  SavedView sv;
  int H, V, n_vt;
  int c0, C;     // chunk start (compact rows) and chunk capacity (multiple of 256)
  int64_t ldc;
  int64_t ldz;   // dZ row pitch (V rounded up to 256, + kPitchPad)
  uint16_t* dZ;  // [C][ldz] token-major: A of dX = dZ W, B of dW^T = X_c^T dZ
  int* queue;  // tile-queue counters of this launch (zero before it)
  int steal;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 pairs: (__bf16)x rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950)
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// kEntGrad: whether the entropy term of dz is formed. Without it (metric-only
// entropy, or no entropy) cb = 0 and dz = p ca' (+ g_lp at the target), one
// FMA per logit fewer, with the same bits.
template <int SHIFT, bool kEntGrad>
__global__ __launch_bounds__(kThreads, 1) void k_dz_tiles(DzParams P) {
  LMH_DECLARE_RING;

  const int n_kept = P.sv.hdr->n_kept;
  const int rows = min(P.C, n_kept - P.c0);
  if (rows <= 0) return;
  const int mt = P.n_vt;
  const int nt = (rows + kBN - 1) / kBN;
  const int ntiles = mt * nt;
  const int tid = threadIdx.x;
  const int nk = P.H / kBK;

  TileQueue q(P.queue, ntiles, P.steal);
  TileClock clk;
  for (;;) {
    const int t = q.next(ring.b[bcast_slot<SHIFT>()]);
    if (t < 0) break;
    clk.tile_start();
    int tm, tn;
    tile_coords<LMH_GM_DZ>(t, mt, nt, tm, tn);

    // coefficients and targets of this lane's eight tokens (columns
    // 16 j + lane % 16 of the wave's 128), loaded before the main loop so that
    // their latency is hidden under it
    float4 rcv[8];
    int tgt[8];
    {
      const int c = P.c0 + tn * kBN + (wave_fresh() & 1) * 128 + (lane_fresh() & 15);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rcv[j] = P.rc[c + j * 16];
        tgt[j] = P.tg[c + j * 16];
      }
    }

    ASrc A;
    BSrc B;
    A.init(P.W + (int64_t)tm * kBM * P.H, P.H, P.V - tm * kBM);
    B.init(P.XcT + (int64_t)tn * kBN, P.ldc, P.H, rows - tn * kBN);
    Acc acc;
    mainloop<SHIFT>(A, B, nk, ring, acc);
    clk.main_done();
    q.claim_ahead();
    // per-tile lane values (see lane_fresh): nothing lane-derived is hoisted
    // out of the tile loop to be spilled across the main loop
    const int lane = lane_fresh(), wave = wave_fresh();
    const int wm = wave >> 1, wn = wave & 1;

    const int vbase = tm * kBM + wm * 128;
    const int fence = acc_read_fence();
    // Tokens past the kept rows have zero coefficients and a zero logit, so
    // their dz is exactly 0. Vocabulary rows at or past V are not masked: those
    // columns of dZ hold finite values that no consumer uses (dX = dZ W reads
    // W rows at or past V as zero; dW^T never stores columns at or past V).
    //
    // dZ leaves through LDS: a lane's registers hold, per token, runs of 4
    // consecutive vocabulary entries (rows 16 i + 4 (lane / 16) + 0..3), so
    // direct stores would write 8-byte pieces. Each wave stages 32 tokens x
    // 128 entries (two column blocks j, 8 KiB: a private quarter of ring slot
    // 0) and stores them back in row order, four 256-byte row segments per
    // instruction. Staging layout: token t (0..31) at t * 256 bytes, its
    // 16-byte chunk q (8 entries) at chunk q ^ (t & 15), so both the
    // register-order writes (32 lanes: 16 tokens x 2 halves of a chunk) and
    // the row-order reads are free of bank conflicts. A wave's LDS accesses
    // are performed in order, so the region is reused for every pair of
    // column blocks without a barrier.
    lds_barrier();  // every wave is done reading the ring
    char* stage = ring.a[0] + wave * 8192;
    const int g = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int j = 2 * jj + jh;
        const float4 k = rcv[j];  // {LSE log2 e, ca - cb LSE, cb, g_lp}
        const int local = tgt[j] - vbase;
        const bool hit = local >= 0 && local < 128 && ((local >> 2) & 3) == g;
        const int want = (local >> 4) * 4 + (local & 3);  // i * 4 + r of the target
        const int t = 16 * jh + (lane & 15);  // this lane's token in the staged 32
        // byte offset of the lane's 8 bytes for row block i: half (g & 1) of
        // chunk q = 2 i + g / 2 at chunk q ^ (t & 15) of row t. Bits 5..7 hold
        // (q >> 1) ^ ((lane >> 1) & 7) and nothing else does, so block i is
        // block 0's offset XOR (i << 5)
        const int off0 = t * 256 + (g & 1) * 8 + ((((g >> 1) ^ lane) & 1) << 4) + ((lane & 14) << 4);
        // the column's 32 entries first, as one straight run (no branch
        // between row blocks, so their chains interleave)
        float d[32];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc_read(acc[i][j][r], fence);
            const float p = __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -k.x));
            d[i * 4 + r] = kEntGrad ? p * fmaf(k.z, z, k.y) : p * k.y;
          }
        // the one-hot term of the target, in the one lane that holds it
        // (added before the rounding to bf16, as for every other term)
        if (hit) {
#pragma unroll
          for (int e = 0; e < 32; ++e)
            if (want == e) d[e] += k.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // entries 16 i + 4 g + 0..3
          const bf16x2_t lo = {(__bf16)d[i * 4 + 0], (__bf16)d[i * 4 + 1]};
          const bf16x2_t hi = {(__bf16)d[i * 4 + 2], (__bf16)d[i * 4 + 3]};
          *reinterpret_cast<uint2*>(stage + (off0 ^ (i << 5))) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
        // one column block at a time (bounds the live copies)
        __builtin_amdgcn_sched_barrier(0);
      }
      // rows 4 u .. 4 u + 3 of the 32 per instruction, 16 lanes a row
      const int q = lane & 15;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int tr = 4 * u + (lane >> 4);
        const uint4 x = *reinterpret_cast<const uint4*>(stage + tr * 256 + ((q ^ (tr & 15)) << 4));
        const int c = tn * kBN + wn * 128 + jj * 32 + tr;  // chunk row
        // non-temporal: 4 GiB of dZ streams past the caches the operand panels use
        const u32x4_t v = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(P.dZ + (int64_t)c * P.ldz + vbase + q * 8));
      }
    }
    clk.tile_done();
  }
  clk.flush(kClkDz);
}

// dX[kept rows] = dZ W: M = chunk rows (A = dZ rows), N = H (B = W: k = v
// rows, h contiguous), K = vocab.
struct DxParams {
  const uint16_t* dZ;  // [C][ldz]
  const uint16_t* W;   // [V][H]
  SavedView sv;
  int H, V;
  int c0, C;
  int64_t ldz;
  float* dX;
  int* queue;  // tile-queue counters of this launch (zero before it)
  int steal;
  // tail split (see kDxSplitMinV)
  int G;       // grid of the launch running the whole tiles (k_dxdw_tiles): its tiles past
               // the last whole round are the tail
  int S;       // pieces per split tail tile (1: never split)
  int rmax;    // largest tail that is split; `part` holds rmax * S tiles
  int kp;      // vocabulary rows per piece, a multiple of 64
  int pieces;  // 0: the whole tiles (and an unsplit tail), 1: the pieces of a split tail
  float* part;  // [rmax * S][256][256] partial tiles, piece p of tail tile r at p * R + r
};

// The tail of a dX launch, from the kept-row count on the device.
struct DxTail {
  int T, R, full;
  bool split;
};
__device__ __forceinline__ DxTail dx_tail(const DxParams& P, int rows) {
  DxTail d;
  const int mt = (rows + kBM - 1) / kBM;
  d.T = mt * ((P.H + kBN - 1) / kBN);
  d.R = d.T % P.G;
  d.split = P.S > 1 && d.R > 0 && d.R <= P.rmax;
  d.full = d.split ? d.T - d.R : d.T;
  return d;
}

template <int SHIFT>
__device__ __forceinline__ void dx_tile_loop(const DxParams& P, const Ring& ring) {
  const int n_kept = P.sv.hdr->n_kept;
  const int rows = min(P.C, n_kept - P.c0);
  if (rows <= 0) return;
  const int mt = (rows + kBM - 1) / kBM;
  const int nt = (P.H + kBN - 1) / kBN;
  const DxTail tail = dx_tail(P, rows);
  // whole tiles, or the S pieces of each split tail tile (unit u: piece u / R
  // of tail tile u % R, so concurrent pieces share their K range)
  const int nunits = P.pieces ? (tail.split ? tail.R * P.S : 0) : tail.full;
  if (nunits == 0) return;
  const int tid = threadIdx.x;
  const int nk = P.pieces ? P.kp / kBK : (P.V + kBK - 1) / kBK;  // W reads zero past V
  const int32_t* kidx = P.sv.kept_idx + P.c0;

  TileQueue q(P.queue, nunits, P.steal);
  TileClock clk;
  for (;;) {
    const int u = q.next(ring.b[bcast_slot<SHIFT>()]);
    if (u < 0) break;
    clk.tile_start();
    int t = u, k0 = 0;
    if (P.pieces) {
      t = tail.full + u % tail.R;
      k0 = (u / tail.R) * P.kp;
    }
    int tm, tn;
    tile_coords<LMH_GM_DX>(t, mt, nt, tm, tn);

    ASrc A;
    BSrc B;
    // a piece reads dZ columns and W rows [k0, k0 + kp): W rows at or past V
    // read as zero, so dZ entries past V (finite) add nothing
    A.init(P.dZ + (int64_t)tm * kBM * P.ldz + k0, P.ldz, rows - tm * kBM);
    B.init(P.W + (int64_t)k0 * P.H + (int64_t)tn * kBN, P.H,
           P.pieces ? min(P.kp, P.V - k0) : P.V, P.H - tn * kBN);
    // original positions of the wave's 128 rows (m0 + lane and m0 + 64 +
    // lane), loaded before the main loop: the epilogue takes each row's from
    // these by lane index instead of waiting on a load per stored row
    int krow[2];
    {
      const int m = tm * kBM + (wave_fresh() >> 1) * 128 + lane_fresh();
#pragma unroll
      for (int h = 0; h < 2; ++h)
        krow[h] = (!P.pieces && m + 64 * h < rows) ? kidx[m + 64 * h] : 0;
    }
    Acc acc;
    mainloop<SHIFT>(A, B, nk, ring, acc);
    clk.main_done();
    q.claim_ahead();
    // per-tile lane values (see lane_fresh): nothing lane-derived is hoisted
    // out of the tile loop to be spilled across the main loop
    const int lane = lane_fresh(), wave = wave_fresh();
    const int wm = wave >> 1, wn = wave & 1;

    // dX rows leave through LDS: a lane holds, per register, one column of a
    // row (row 16 i + 4 (lane / 16) + r, column 16 j + lane % 16), so direct
    // stores would write 4-byte pieces. Each wave stages the 16 rows x 128
    // columns of one row block i (8 KiB, a private quarter of ring slot 0;
    // row t at t * 512 bytes, 16-byte chunk q at chunk q ^ t) and stores whole
    // 512-byte row segments, two rows per instruction, looking up each row's
    // position once. The writes (4 rows x 16 columns per instruction) and the
    // row reads are free of bank conflicts.
    const int fence = acc_read_fence();
    lds_barrier();  // every wave is done reading the ring
    float* stage = reinterpret_cast<float*>(ring.a[0] + wave * 8192);
    const int m0 = tm * kBM + wm * 128;  // first chunk row of the wave's block
    const int n0 = tn * kBN + wn * 128;  // first h of the wave's block
    const int g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = j * 16 + (lane & 15);
          stage[t * 128 + (((col >> 2) ^ t) << 2) + (col & 3)] = acc_read(acc[i][j][r], fence);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const int q = lane & 31;  // 16-byte chunk of the row
#pragma unroll
      for (int uu = 0; uu < 8; ++uu) {
        const int t = 2 * uu + (lane >> 5);
        const int m = m0 + i * 16 + t;
        const int h = n0 + q * 4;
        const float4 x = *reinterpret_cast<const float4*>(stage + t * 128 + ((q ^ t) << 2));
        // the row's position: wave row i * 16 + 2 uu for lanes 0..31, the
        // next one for lanes 32..63 (compile-time lanes of krow)
        const int rr = i * 16 + 2 * uu;
        const int plo = __builtin_amdgcn_readlane(krow[i >> 2], rr & 63);
        const int phi = __builtin_amdgcn_readlane(krow[i >> 2], (rr + 1) & 63);
        const int pos = (lane >> 5) ? phi : plo;
        if (P.pieces)  // the whole partial tile, row-major
          *reinterpret_cast<float4*>(P.part + (int64_t)u * (kBM * kBN) +
                                     (m - tm * kBM) * kBN + (h - tn * kBN)) = x;
        else if (m < rows && h < P.H)  // H is a multiple of 4: a chunk is whole
          *reinterpret_cast<float4*>(P.dX + (int64_t)pos * P.H + h) = x;
      }
    }
    clk.tile_done();
  }
  clk.flush(kClkDx);
}

// A split tail's pieces, as a launch of their own (dX's whole tiles run in
// k_dxdw_tiles, ahead of dW).
template <int SHIFT>
__global__ __launch_bounds__(kThreads, 1) void k_dx_tiles(DxParams P) {
  LMH_DECLARE_RING;
  dx_tile_loop<SHIFT>(P, ring);
}

// The split tail's dX tiles: the S partial tiles of each are summed in piece
// order (a fixed order, so results are reproducible) and scattered to the
// rows' original positions. One thread per 16-byte chunk of a tile row.
__global__ __launch_bounds__(256) void k_dx_reduce(DxParams P) {
  const int n_kept = P.sv.hdr->n_kept;
  const int rows = min(P.C, n_kept - P.c0);
  if (rows <= 0) return;
  const DxTail tail = dx_tail(P, rows);
  if (!tail.split) return;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  constexpr int kChunks = kBN / 4;
  if (idx >= (int64_t)tail.R * kBM * kChunks) return;
  const int r = (int)(idx / (kBM * kChunks));
  const int e = (int)(idx % (kBM * kChunks));
  const int row = e / kChunks, q = e % kChunks;
  int tm, tn;
  tile_coords<LMH_GM_DX>(tail.full + r, (rows + kBM - 1) / kBM, (P.H + kBN - 1) / kBN, tm, tn);
  const int m = tm * kBM + row, h = tn * kBN + q * 4;
  if (m >= rows || h >= P.H) return;
  const float* src = P.part + (int64_t)r * (kBM * kBN) + row * kBN + q * 4;
  float4 acc = *reinterpret_cast<const float4*>(src);
  for (int p = 1; p < P.S; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(src + (int64_t)p * tail.R * (kBM * kBN));
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *reinterpret_cast<float4*>(P.dX + (int64_t)P.sv.kept_idx[P.c0 + m] * P.H + h) = acc;
}

// dW^T (+)= X_c^T dZ: M = H (A = X_c^T rows), N = vocab (B = dZ: k = chunk
// rows, vocabulary contiguous), K = chunk rows; stored transposed into dW.
struct DwParams {
  const uint16_t* XcT;  // [H][ldc]: the chunk's kept rows, transposed
  const uint16_t* dZ;   // [C][ldz]
  const SavedHeader* hdr;
  int H, V;
  int c0, C;
  int64_t ldc, ldz;
  int accumulate;
  float* dW;
  int* queue;  // tile-queue counters of this launch (zero before it)
  int steal;
};

template <int SHIFT>
__device__ __forceinline__ void dw_tile_loop(const DwParams& P, const Ring& ring, int rows, int nk) {
  const int mt = (P.H + kBM - 1) / kBM;
  const int nt = (P.V + kBN - 1) / kBN;
  const int ntiles = mt * nt;
  const int tid = threadIdx.x;

  TileQueue q(P.queue, ntiles, P.steal);
  TileClock clk;
  for (;;) {
    const int t = q.next(ring.b[bcast_slot<SHIFT>()]);
    if (t < 0) break;
    clk.tile_start();
    int tm, tn;
    tile_coords<LMH_GM_DW>(t, mt, nt, tm, tn);

    ASrc A;
    BSrc B;
    A.init(P.XcT + (int64_t)tm * kBM * P.ldc, P.ldc, P.H - tm * kBM);
    B.init(P.dZ + (int64_t)tn * kBN, P.ldz, rows, kBN);  // ldz covers every v of the tile
    Acc acc;
    mainloop<SHIFT>(A, B, nk, ring, acc);
    clk.main_done();
    q.claim_ahead();
    // per-tile lane values (see lane_fresh): nothing lane-derived is hoisted
    // out of the tile loop to be spilled across the main loop
    const int lane = lane_fresh(), wave = wave_fresh();
    const int wm = wave >> 1, wn = wave & 1;

    // dW leaves through LDS the way dZ does in k_dz_tiles. A lane holds, per
    // vocabulary row 16 j + lane % 16, runs of 4 consecutive h (16 i +
    // 4 (lane / 16) + 0..3): one 16-byte chunk of the row. Each wave stages
    // the 16 vocabulary rows x 128 h of one column block j (8 KiB, a private
    // quarter of ring slot 0; row t at t * 512 bytes, chunk q at chunk q ^ t)
    // and stores two 512-byte row segments per instruction.
    const int fence = acc_read_fence();
    lds_barrier();  // every wave is done reading the ring
    char* stage = ring.a[0] + wave * 8192;
    const int h0 = tm * kBM + wm * 128;  // first h of the wave's rows
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // rows 2 u, 2 u + 1 of the block per store instruction, 32 lanes a row
      const int q = lane & 31;
      const int h = h0 + q * 4;
      // accumulating: the block's previous values, all eight loads issued
      // before the staging so that one wait covers them
      float4 old[8];
      if (P.accumulate) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int v = tn * kBN + wn * 128 + j * 16 + 2 * u + (lane >> 5);
          old[u] = (v < P.V && h < P.H)
                       ? *reinterpret_cast<const float4*>(P.dW + (int64_t)v * P.H + h)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      const int t = lane & 15;  // this lane's vocabulary row in the wave's block
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i * 4 + g;  // h = 4 q .. 4 q + 3 of the wave's 128
        const float4 x = make_float4(
            acc_read(acc[i][j][0], fence), acc_read(acc[i][j][1], fence),
            acc_read(acc[i][j][2], fence), acc_read(acc[i][j][3], fence));
        *reinterpret_cast<float4*>(stage + t * 512 + ((q ^ t) << 4)) = x;
      }
      __builtin_amdgcn_sched_barrier(0);
      // the block's eight row pieces read back together (the reads stay in
      // the wave's region whatever the bounds, so one wait covers them), then
      // stored where the row and h exist
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int tr = 2 * u + (lane >> 5);
        x[u] = *reinterpret_cast<const float4*>(stage + tr * 512 + ((q ^ tr) << 4));
      }
      if (P.accumulate) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          x[u].x += old[u].x;
          x[u].y += old[u].y;
          x[u].z += old[u].z;
          x[u].w += old[u].w;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = tn * kBN + wn * 128 + j * 16 + 2 * u + (lane >> 5);
        if (v < P.V && h < P.H) {  // H is a multiple of 4: a chunk is whole
          const f32x4_t o = {x[u].x, x[u].y, x[u].z, x[u].w};
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4_t*>(P.dW + (int64_t)v * P.H + h));
        }
      }
    }
    clk.tile_done();
  }
  clk.flush(kClkDw);
}

// K of dW is the chunk's kept rows, a count only the device has (the saved
// header): the kernel takes the instance whose stage shift runs exactly that
// many stages, where a shift chosen on the host from the chunk capacity ran
// up to 11 padding stages per tile (at 23 % kept rows, 11 of 128).
__device__ __forceinline__ void dw_phase(const DwParams& P, const Ring& ring) {
  const int n_kept = P.hdr->n_kept;
  int rows = min(P.C, n_kept - P.c0);
  if (rows <= 0) {
    if (P.accumulate) return;  // nothing to add
    rows = 0;                  // first chunk with no kept rows: write zeros
  }
  const int nk = (rows + kBK - 1) / kBK;  // dZ rows past `rows` read as zero
  switch (shift_for(nk)) {
    case 0: dw_tile_loop<0>(P, ring, rows, nk); break;
    case 2: dw_tile_loop<2>(P, ring, rows, nk); break;
    case 4: dw_tile_loop<4>(P, ring, rows, nk); break;
    case 6: dw_tile_loop<6>(P, ring, rows, nk); break;
    case 8: dw_tile_loop<8>(P, ring, rows, nk); break;
    default: dw_tile_loop<10>(P, ring, rows, nk); break;
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_dw_tiles(DwParams P) {
  LMH_DECLARE_RING;
  dw_phase(P, ring);
}

// dX's whole tiles, then dW, in one launch: a workgroup goes on to dW tiles
// as soon as its dX tiles are done. dX has few long tiles per workgroup (4 of
// 2.7 ms at N 16384, H 4096, V 131072), too few to steal, and the XCDs finish
// them 5-9 % apart; as separate launches every CU waited for the last XCD
// before dW began. (Two streams cannot do this safely: persistent
// workgroups keep a CU until their queue is empty, so dW workgroups placed
// first would hold CUs that dX workgroups need.)
__global__ __launch_bounds__(kThreads, 1) void k_dxdw_tiles(DxParams X, DwParams W) {
  LMH_DECLARE_RING;
  switch (shift_for((X.V + kBK - 1) / kBK)) {
    case 0: dx_tile_loop<0>(X, ring); break;
    case 2: dx_tile_loop<2>(X, ring); break;
    case 4: dx_tile_loop<4>(X, ring); break;
    case 6: dx_tile_loop<6>(X, ring); break;
    case 8: dx_tile_loop<8>(X, ring); break;
    default: dx_tile_loop<10>(X, ring); break;
  }
  // every wave has read the dX queue's last broadcast before the dW queue
  // writes its own (the two may share a word)
  lds_barrier();
  dw_phase(W, ring);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static int g_cu_count[64];

static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cu_count[dev];
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return n;
}

// Persistent grid: at most one workgroup per CU, a multiple of the XCD count.
static int persistent_grid(int64_t max_tiles) {
  int64_t g = cu_count();
  g = g / kXcds * kXcds;
  if (g < kXcds) g = kXcds;
  int64_t need = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (need < kXcds) need = kXcds;
  return (int)(need < g ? need : g);
}

// Tile stealing between XCDs pays only when a tile is a small part of a
// workgroup's work.
static inline int steal_for(int64_t tiles, int grid) { return tiles >= 16 * (int64_t)grid; }

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static int check_sizes(int64_t N, int64_t H, int64_t V) {
  if (N < 0 || H <= 0 || V <= 0) return LMHEAD_ERR_INVALID_ARG;
  if (H % 64 != 0) return LMHEAD_ERR_UNSUPPORTED;
  if (N > kMaxN || H > kMaxH || V > kMaxV) return LMHEAD_ERR_UNSUPPORTED;  // see kMaxN
  return LMHEAD_OK;
}

// Optional per-kernel timing (benchmarks only): hipEvent pairs recorded on
// the launch stream around every launch while profiling is on.
enum KernelKind {
  KK_COMPACT = 0, KK_GATHER_COLS, KK_FWD, KK_MERGE, KK_ZERO_SKIPPED, KK_ZERO_ROWS,
  KK_DZ, KK_DX, KK_DW, KK_ZERO_QUEUES, KK_BWD_ROWS, KK_MERGE_SHARDS, KK_DX_REDUCE, KK_DXDW,
  KK_COUNT
};
static const char* const kKernelNames[KK_COUNT] = {
    "compact",   "gather_cols", "fwd_tiles", "merge",    "zero_skipped",
    "zero_rows", "dz_tiles",    "dx_tiles",  "dw_tiles", "zero_queues", "bwd_rows",
    "merge_shards", "dx_reduce", "dxdw_tiles"};

struct ProfRec {
  hipEvent_t a, b;
  int kind;
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
// Set for the duration of an allocation-free call: its launches create no
// timing events (event creation allocates).
static thread_local bool t_no_events = false;
static std::vector<ProfRec> g_prof_recs;
static std::vector<hipEvent_t> g_prof_pool;

static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launches kernel `k` with the given configuration on stream s; returns a
// lmhead_status (LMHEAD_ERR_HIP if this launch failed). Records timing events
// when profiling is on.
template <typename... KArgs, typename... Args>
static int launch(int kind, void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                  Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (g_prof_on && !t_no_events) {
      a = prof_event();
      b = prof_event();
    }
  }
  if (a && b && hipEventRecord(a, s) != hipSuccess) return LMHEAD_ERR_HIP;
  if (lmh_launch::launch_kernel(k, grid, block, s, args...) != hipSuccess) return LMHEAD_ERR_HIP;
  if (a && b) {
    if (hipEventRecord(b, s) != hipSuccess) return LMHEAD_ERR_HIP;
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_recs.push_back(ProfRec{a, b, kind});
  }
  return LMHEAD_OK;
}

// Launches the instance of a GEMM kernel for the stage shift (even, 0..10)
// that makes its stage count run without padding (mainloop).
template <class Params, class... Kernels>
static int launch_shifted(int kind, int shift, dim3 grid, hipStream_t s, const Params& p,
                          Kernels... k) {
  void (*table[])(Params) = {k...};
  static_assert(sizeof...(Kernels) == 6, "one instance per even shift");
  return launch(kind, table[shift / 2], grid, dim3(kThreads), s, p);
}



#define LMH_TRY(expr)                  \
  do {                                 \
    const int st_ = (expr);            \
    if (st_ != LMHEAD_OK) return st_;  \
  } while (0)

}  // namespace lmh

using namespace lmh;

LMH_API size_t lmhead_saved_bytes(int64_t N) {
  if (N < 0) return 0;
  return saved_bytes_for(N);
}

LMH_API size_t lmhead_fwd_workspace_bytes(int64_t N, int64_t H, int64_t V) {
  if (check_sizes(N, H, V) != LMHEAD_OK) return 0;
  return fwd_ws(N, H, V).total;
}

LMH_API size_t lmhead_bwd_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t token_chunk) {
  if (check_sizes(N, H, V) != LMHEAD_OK) return 0;
  return bwd_ws(N, H, V, token_chunk).total;
}

// The forward for the whole vocabulary (rec == nullptr) or for the shard of
// rows [vocab_start, vocab_start + V) of a vocabulary of V_total entries
// (rec != nullptr: per-row shard statistics instead of log-prob / entropy).
static int fwd_impl(const void* hidden, const void* weight, const int32_t* targets,
                    const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V, int64_t vocab_start,
                    int64_t V_total, int flags, int block, float* logp, float* entropy,
                    float4* rec, void* saved, size_t saved_bytes, void* workspace,
                    size_t workspace_bytes, hipStream_t s) {
  const FwdWs L = fwd_ws(N, H, V);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return LMHEAD_ERR_WORKSPACE;
  if (saved_bytes < saved_bytes_for(N)) return LMHEAD_ERR_WORKSPACE;
  SavedView sv = saved_view(saved, N);
  char* w = static_cast<char*>(workspace);
  int32_t* tg = reinterpret_cast<int32_t*>(w + L.tg);
  // the target-logit array is the compaction's scratch until the projection writes it
  int* cscratch = reinterpret_cast<int*>(w + L.zt);
  const int nch = compact_chunks(N);
  if (nch > 0)
    LMH_TRY(launch(KK_COMPACT, k_compact_count, dim3(nch), dim3(kCompactThreads), s, keep_mask,
                   targets, (int)N, (int)V_total, block, cscratch, nch));
  LMH_TRY(launch(KK_COMPACT, k_compact_scan, dim3(1), dim3(kScanThreads), s, cscratch, nch,
                 (int)N, (int)H, (int)V_total, flags, sv.hdr));
  if (N == 0) return LMHEAD_OK;
  LMH_TRY(launch(KK_COMPACT, k_compact_write, dim3(nch), dim3(kCompactThreads), s, keep_mask,
                 targets, (int)N, block, (const int*)cscratch, (const SavedHeader*)sv.hdr,
                 sv.kept_idx, sv.pos, tg, (int)tile_rows(N), (int)vocab_start));

  const int nv = n_vtiles(V);
  const int64_t ldc = ldc_of(N);
  uint16_t* XcT = reinterpret_cast<uint16_t*>(w + L.xct);
  LMH_TRY(launch(KK_GATHER_COLS, k_gather_cols, dim3((unsigned)(ldc / kTp), (unsigned)(H / kTp)),
                 dim3(256), s, static_cast<const uint16_t*>(hidden), (const SavedHeader*)sv.hdr,
                 (const int32_t*)sv.kept_idx, 0, (int)H, XcT, ldc));

  FwdParams P;
  P.W = static_cast<const uint16_t*>(weight);
  P.XcT = XcT;
  P.ldc = ldc;
  P.tg = tg;
  P.hdr = sv.hdr;
  P.H = (int)H;
  P.V = (int)V;
  P.n_vt = nv;
  P.ldp = N;
  P.zt = reinterpret_cast<float*>(w + L.zt);
  P.pm = reinterpret_cast<float*>(w + L.pm);
  P.ps = reinterpret_cast<float*>(w + L.ps);
  P.pb = reinterpret_cast<float*>(w + L.pb);
  const int64_t max_tiles = (int64_t)nv * ((N + kBN - 1) / kBN);
  const int grid = persistent_grid(max_tiles);
  P.queue = reinterpret_cast<int*>(w + L.q);
  P.steal = steal_for(max_tiles, grid);
  LMH_TRY(launch(KK_ZERO_QUEUES, k_zero_ints, dim3(1), dim3(64), s, P.queue, kQueueInts));
  LMH_TRY(launch_shifted(KK_FWD, stage_shift((int)(H / kBK)), dim3(grid), s, P,
                         k_fwd_tiles<0>, k_fwd_tiles<2>, k_fwd_tiles<4>, k_fwd_tiles<6>,
                         k_fwd_tiles<8>, k_fwd_tiles<10>));

  const dim3 mgrid((unsigned)((N + kMergeRows - 1) / kMergeRows));
  const dim3 rgrid((unsigned)((N + 255) / 256));
  if (rec) {
    LMH_TRY(launch(KK_MERGE, k_merge<true>, mgrid, dim3(256), s, (const float*)P.pm,
                   (const float*)P.ps, (const float*)P.pb, (const float*)P.zt, (int64_t)N, nv,
                   (const int32_t*)tg, (int)V, sv, (float*)nullptr, (float*)nullptr, rec));
    LMH_TRY(launch(KK_ZERO_SKIPPED, k_skipped_records, rgrid, dim3(256), s,
                   (const int32_t*)sv.pos, (int)N, rec));
  } else {
    LMH_TRY(launch(KK_MERGE, k_merge<false>, mgrid, dim3(256), s, (const float*)P.pm,
                   (const float*)P.ps, (const float*)P.pb, (const float*)P.zt, (int64_t)N, nv,
                   (const int32_t*)tg, (int)V, sv, logp, entropy, (float4*)nullptr));
    LMH_TRY(launch(KK_ZERO_SKIPPED, k_zero_skipped, rgrid, dim3(256), s, (const int32_t*)sv.pos,
                   (int)N, logp, entropy));
  }
  return LMHEAD_OK;
}

// Shared by the two whole-vocabulary forwards: block = 1 compacts to the kept
// rows, block = kBlockSparseRows lists whole row tiles (flag bit 2 records it).
constexpr int kBlockSparseRows = kBN;  // one GEMM token tile
static int fwd_entry(const void* hidden, const void* weight, const int32_t* targets,
                     const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
                     int return_entropy, int entropy_requires_grad, float* logp, float* entropy,
                     void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                     void* stream, int block) {
  int st = check_sizes(N, H, V);
  if (st != LMHEAD_OK) return st;
  if (!saved) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (!hidden || !weight || !targets || !logp)) return LMHEAD_ERR_INVALID_ARG;
  if (!weight) return LMHEAD_ERR_INVALID_ARG;
  // an empty output may have a NULL address, so presence is only checked for N > 0
  if (N > 0 && (return_entropy != 0) != (entropy != nullptr)) return LMHEAD_ERR_INVALID_ARG;
  if (entropy_requires_grad && !return_entropy) return LMHEAD_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(saved) || !aligned16(workspace))
    return LMHEAD_ERR_INVALID_ARG;
  // this call merges the vocabulary tiles itself, so its LSE and entropy are complete
  const int flags = (return_entropy ? kFlagReturnEntropy : 0) |
                    (entropy_requires_grad ? kFlagEntropyGrad : 0) |
                    (block > 1 ? kFlagBlockSparse : 0) | kFlagComplete;
  return fwd_impl(hidden, weight, targets, keep_mask, N, H, V, 0, V, flags, block, logp, entropy,
                  nullptr, saved, saved_bytes, workspace, workspace_bytes,
                  static_cast<hipStream_t>(stream));
}

LMH_API int lmhead_fwd(const void* hidden, const void* weight, const int32_t* targets,
                       const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
                       int return_entropy, int entropy_requires_grad, float* logp, float* entropy,
                       void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return fwd_entry(hidden, weight, targets, keep_mask, N, H, V, return_entropy,
                   entropy_requires_grad, logp, entropy, saved, saved_bytes, workspace,
                   workspace_bytes, stream, 1);
}

LMH_API int lmhead_fwd_blocksparse(const void* hidden, const void* weight,
                                   const int32_t* targets, const uint8_t* keep_mask, int64_t N,
                                   int64_t H, int64_t V, int return_entropy,
                                   int entropy_requires_grad, float* logp, float* entropy,
                                   void* saved, size_t saved_bytes, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return fwd_entry(hidden, weight, targets, keep_mask, N, H, V, return_entropy,
                   entropy_requires_grad, logp, entropy, saved, saved_bytes, workspace,
                   workspace_bytes, stream, kBlockSparseRows);
}

// ---------------------------------------------------------------------------
// Allocation-free forward: lmhead_fwd with its workspace in a file-scope
// device array, for callers that cannot allocate. Host code never names the
// array as an address (its host-side name is a stand-in); the device address
// comes from hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = LMHEAD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on its first use).
static int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LMHEAD_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return LMHEAD_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LMHEAD_OK;
}

LMH_API int lmhead_fwd_noalloc(const void* hidden, const void* weight, const int32_t* targets,
                               const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
                               int return_entropy, int entropy_requires_grad, float* logp,
                               float* entropy, void* saved, size_t saved_bytes, void* stream) {
  const int st = check_sizes(N, H, V);
  if (st != LMHEAD_OK) return st;
  if (fwd_ws(N, H, V).total > kNoAllocScratchBytes) return LMHEAD_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = noalloc_scratch(&ws);
  if (sst != LMHEAD_OK) return sst;
  struct NoEvents {
    NoEvents() { t_no_events = true; }
    ~NoEvents() { t_no_events = false; }
  } no_events;
  // the tile-queue counters in the scratch are zeroed by a kernel each call;
  // every other workspace entry the kernels read is written earlier in the call
  return fwd_entry(hidden, weight, targets, keep_mask, N, H, V, return_entropy,
                   entropy_requires_grad, logp, entropy, saved, saved_bytes, ws,
                   kNoAllocScratchBytes, stream, 1);
}

LMH_API int lmhead_fwd_partial(const void* hidden, const void* weight_shard,
                               const int32_t* targets, const uint8_t* keep_mask, int64_t N,
                               int64_t H, int64_t V_shard, int64_t vocab_start, int64_t V_total,
                               float* partial, void* saved, size_t saved_bytes,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_sizes(N, H, V_shard);
  if (st != LMHEAD_OK) return st;
  if (vocab_start < 0 || V_total > kMaxV || vocab_start + V_shard > V_total)
    return LMHEAD_ERR_INVALID_ARG;
  if (!saved || !weight_shard) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (!hidden || !targets || !partial)) return LMHEAD_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight_shard) || !aligned16(saved) ||
      !aligned16(workspace) || !aligned16(partial))
    return LMHEAD_ERR_INVALID_ARG;
  return fwd_impl(hidden, weight_shard, targets, keep_mask, N, H, V_shard, vocab_start, V_total,
                  0, 1, nullptr, nullptr, reinterpret_cast<float4*>(partial), saved, saved_bytes,
                  workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

LMH_API int lmhead_merge_partials(const float* partials, int64_t P, int64_t N,
                                  int return_entropy, int entropy_requires_grad, float* logp,
                                  float* entropy, void* saved, size_t saved_bytes,
                                  void* stream) {
  if (P < 1 || P > 65536 || N < 0 || N > kMaxN) return LMHEAD_ERR_INVALID_ARG;
  if (!saved) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (!partials || !logp)) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (return_entropy != 0) != (entropy != nullptr)) return LMHEAD_ERR_INVALID_ARG;
  if (entropy_requires_grad && !return_entropy) return LMHEAD_ERR_INVALID_ARG;
  if (!aligned16(partials) || !aligned16(saved)) return LMHEAD_ERR_INVALID_ARG;
  if (saved_bytes < saved_bytes_for(N)) return LMHEAD_ERR_WORKSPACE;
  const int flags = (return_entropy ? kFlagReturnEntropy : 0) |
                    (entropy_requires_grad ? kFlagEntropyGrad : 0);
  SavedView sv = saved_view(saved, N);
  const unsigned blocks = (unsigned)(N > 0 ? (N + 255) / 256 : 1);
  return launch(KK_MERGE_SHARDS, k_merge_shards, dim3(blocks), dim3(256),
                static_cast<hipStream_t>(stream), reinterpret_cast<const float4*>(partials),
                (int)P, N, sv, flags, logp, entropy);
}

// The backward for the whole vocabulary (vocab_start = 0) or for the shard of
// rows [vocab_start, vocab_start + V) (grad_weight is then the shard's rows
// and grad_hidden this shard's share of dX).
static int bwd_impl(const void* hidden, const void* weight, const int32_t* targets, int64_t N,
                    int64_t H, int64_t V, int64_t vocab_start, bool shard,
                    int entropy_requires_grad, const void* saved, size_t saved_bytes,
                    const float* grad_logp, const float* grad_entropy, float* grad_hidden,
                    float* grad_weight, int64_t token_chunk, void* workspace,
                    size_t workspace_bytes, hipStream_t s) {
  if (saved_bytes < saved_bytes_for(N)) return LMHEAD_ERR_WORKSPACE;
  const BwdWs L = bwd_ws(N, H, V, token_chunk);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return LMHEAD_ERR_WORKSPACE;
  const BwdGeom G = bwd_geom(N, V, token_chunk);

  char* w = static_cast<char*>(workspace);
  // Every kernel below reads the kept-row count from the checked copy of the
  // saved header (k_bwd_check), never from the saved header itself.
  SavedHeader* chk = reinterpret_cast<SavedHeader*>(w + L.chk);
  SavedView sv = saved_view(const_cast<void*>(saved), N);
  LMH_TRY(launch(KK_BWD_ROWS, k_bwd_check, dim3(1), dim3(64), s, sv.hdr, (int)N, (int)H, (int)V,
                 (int)vocab_start, (int)shard, entropy_requires_grad, chk));
  sv.hdr = chk;
  uint16_t* XcT = reinterpret_cast<uint16_t*>(w + L.xct);
  uint16_t* dZ = reinterpret_cast<uint16_t*>(w + L.dz);
  const uint16_t* X = static_cast<const uint16_t*>(hidden);
  const uint16_t* Wt = static_cast<const uint16_t*>(weight);
  int* queues = reinterpret_cast<int*>(w + L.q);
  float4* rc = reinterpret_cast<float4*>(w + L.rc);
  int32_t* tg = reinterpret_cast<int32_t*>(w + L.tg);
  LMH_TRY(launch(KK_ZERO_QUEUES, k_zero_ints, dim3((unsigned)((L.nq + 255) / 256)), dim3(256), s,
                 queues, (int)L.nq));

  if (N > 0) {
    const int nrows = (int)tile_rows(N);
    LMH_TRY(launch(KK_BWD_ROWS, k_bwd_rows, dim3((unsigned)(nrows / 256)), dim3(256), s, sv,
                   targets, grad_logp, entropy_requires_grad ? grad_entropy : nullptr, nrows,
                   (int)vocab_start, rc, tg));
    LMH_TRY(launch(KK_ZERO_ROWS, k_zero_rows,
                   dim3((unsigned)std::min<int64_t>(N, kZeroRowsGrid)), dim3(256), s,
                   (const int32_t*)sv.pos, (const SavedHeader*)chk, (int)N, (int)H, grad_hidden));
  }
  const int nv = n_vtiles(V);
  const int64_t nchunks = N > 0 ? (N + G.C - 1) / G.C : 1;
  auto dw_params = [&](int64_t ch, int c0) {
    DwParams Wp;
    Wp.XcT = XcT;
    Wp.dZ = dZ;
    Wp.hdr = sv.hdr;
    Wp.H = (int)H;
    Wp.V = (int)V;
    Wp.c0 = c0;
    Wp.C = (int)G.C;
    Wp.ldc = G.ldc;
    Wp.ldz = G.ldz;
    Wp.accumulate = ch > 0;
    Wp.dW = grad_weight;
    Wp.queue = queues + (ch * kBwdQueueSets + 3) * kQueueInts;
    Wp.steal = 0;
    return Wp;
  };
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int c0 = (int)(ch * G.C);
    if (N > 0) {
      // this chunk's kept rows, transposed: X_c^T [H][C]
      LMH_TRY(launch(KK_GATHER_COLS, k_gather_cols,
                     dim3((unsigned)(G.C / kTp), (unsigned)(H / kTp)), dim3(256), s, X,
                     (const SavedHeader*)chk, (const int32_t*)sv.kept_idx, c0, (int)H, XcT,
                     G.ldc));
      DzParams D;
      D.W = Wt;
      D.XcT = XcT;
      D.ldc = G.ldc;
      D.rc = rc;
      D.tg = tg;
      D.sv = sv;
      D.H = (int)H;
      D.V = (int)V;
      D.n_vt = nv;
      D.c0 = c0;
      D.C = (int)G.C;
      D.ldz = G.ldz;
      D.dZ = dZ;
      const int64_t dz_tiles = (int64_t)nv * (G.C / kBN);
      const int dz_grid = persistent_grid(dz_tiles);
      D.queue = queues + (ch * kBwdQueueSets + 0) * kQueueInts;
      D.steal = steal_for(dz_tiles, dz_grid);
      const int dz_shift = stage_shift((int)(H / kBK));
      if (entropy_requires_grad)
        LMH_TRY(launch_shifted(KK_DZ, dz_shift, dim3(dz_grid), s, D, k_dz_tiles<0, true>,
                               k_dz_tiles<2, true>, k_dz_tiles<4, true>, k_dz_tiles<6, true>,
                               k_dz_tiles<8, true>, k_dz_tiles<10, true>));
      else
        LMH_TRY(launch_shifted(KK_DZ, dz_shift, dim3(dz_grid), s, D, k_dz_tiles<0, false>,
                               k_dz_tiles<2, false>, k_dz_tiles<4, false>, k_dz_tiles<6, false>,
                               k_dz_tiles<8, false>, k_dz_tiles<10, false>));

      DxParams X2;
      X2.dZ = dZ;
      X2.ldz = G.ldz;
      X2.W = Wt;
      X2.sv = sv;
      X2.H = (int)H;
      X2.V = (int)V;
      X2.c0 = c0;
      X2.C = (int)G.C;
      X2.dX = grad_hidden;
      const int64_t dx_tiles = dx_tiles_per_chunk(G.C, H);
      const int64_t dw_tiles = (int64_t)nv * ((H + kBN - 1) / kBN);
      // one launch runs dX's whole tiles, then dW's tiles: the grid fits both
      const int grid = std::max(persistent_grid(dx_tiles), persistent_grid(dw_tiles));
      X2.queue = queues + (ch * kBwdQueueSets + 1) * kQueueInts;
      X2.steal = steal_for(dx_tiles, grid);
      X2.G = grid;
      X2.S = dx_pieces(V);
      X2.rmax = dx_tail_max(G.C, H, V);
      X2.kp = dx_piece_k(V);
      X2.part = reinterpret_cast<float*>(w + L.part);
      X2.pieces = 0;
      DwParams Wp = dw_params(ch, c0);
      Wp.steal = steal_for(dw_tiles, grid);
      LMH_TRY(launch(KK_DXDW, k_dxdw_tiles, dim3(grid), dim3(kThreads), s, X2, Wp));
      if (X2.S > 1) {
        // the pieces of a split tail, then their sum; both exit at once when
        // the kept rows leave no tail to split (decided on the device)
        X2.pieces = 1;
        const int64_t units = (int64_t)X2.rmax * X2.S;
        const int pgrid = persistent_grid(units);
        X2.queue = queues + (ch * kBwdQueueSets + 2) * kQueueInts;
        X2.steal = steal_for(units, pgrid);
        LMH_TRY(launch_shifted(KK_DX, shift_for(X2.kp / kBK), dim3(pgrid), s, X2, k_dx_tiles<0>,
                               k_dx_tiles<2>, k_dx_tiles<4>, k_dx_tiles<6>, k_dx_tiles<8>,
                               k_dx_tiles<10>));
        LMH_TRY(launch(KK_DX_REDUCE, k_dx_reduce, dim3((unsigned)(X2.rmax * (kBM * kBN / 4) / 256)),
                       dim3(256), s, X2));
      }
    } else {
      // no rows: dW is written as zeros
      const int64_t dw_tiles = (int64_t)nv * ((H + kBN - 1) / kBN);
      const int dw_grid = persistent_grid(dw_tiles);
      DwParams Wp = dw_params(ch, c0);
      Wp.steal = steal_for(dw_tiles, dw_grid);
      LMH_TRY(launch(KK_DW, k_dw_tiles, dim3(dw_grid), dim3(kThreads), s, Wp));
    }
  }
  return LMHEAD_OK;
}

// Argument checks shared by lmhead_bwd and lmhead_bwd_partial.
static int bwd_check(const void* hidden, const void* weight, const int32_t* targets, int64_t N,
                     int entropy_requires_grad, const void* saved, const float* grad_logp,
                     const float* grad_entropy, const float* grad_hidden,
                     const float* grad_weight, const void* workspace) {
  if (!saved || !weight || !grad_weight) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (!hidden || !targets || !grad_logp || !grad_hidden)) return LMHEAD_ERR_INVALID_ARG;
  if (N > 0 && (entropy_requires_grad != 0) != (grad_entropy != nullptr))
    return LMHEAD_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(saved) || !aligned16(workspace) ||
      !aligned16(grad_hidden) || !aligned16(grad_weight))
    return LMHEAD_ERR_INVALID_ARG;
  return LMHEAD_OK;
}

LMH_API int lmhead_bwd(const void* hidden, const void* weight, const int32_t* targets, int64_t N,
                       int64_t H, int64_t V, int entropy_requires_grad, const void* saved,
                       size_t saved_bytes, const float* grad_logp, const float* grad_entropy,
                       float* grad_hidden, float* grad_weight, int64_t token_chunk,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_sizes(N, H, V);
  if (st != LMHEAD_OK) return st;
  st = bwd_check(hidden, weight, targets, N, entropy_requires_grad, saved, grad_logp,
                 grad_entropy, grad_hidden, grad_weight, workspace);
  if (st != LMHEAD_OK) return st;
  return bwd_impl(hidden, weight, targets, N, H, V, 0, false, entropy_requires_grad, saved, saved_bytes,
                  grad_logp, grad_entropy, grad_hidden, grad_weight, token_chunk, workspace,
                  workspace_bytes, static_cast<hipStream_t>(stream));
}

LMH_API int lmhead_bwd_partial(const void* hidden, const void* weight_shard,
                               const int32_t* targets, int64_t N, int64_t H, int64_t V_shard,
                               int64_t vocab_start, int entropy_requires_grad, const void* saved,
                               size_t saved_bytes, const float* grad_logp,
                               const float* grad_entropy, float* grad_hidden,
                               float* grad_weight_shard, int64_t token_chunk, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int st = check_sizes(N, H, V_shard);
  if (st != LMHEAD_OK) return st;
  if (vocab_start < 0 || vocab_start + V_shard > kMaxV) return LMHEAD_ERR_INVALID_ARG;
  st = bwd_check(hidden, weight_shard, targets, N, entropy_requires_grad, saved, grad_logp,
                 grad_entropy, grad_hidden, grad_weight_shard, workspace);
  if (st != LMHEAD_OK) return st;
  return bwd_impl(hidden, weight_shard, targets, N, H, V_shard, vocab_start, true,
                  entropy_requires_grad, saved, saved_bytes, grad_logp, grad_entropy,
                  grad_hidden, grad_weight_shard, token_chunk, workspace, workspace_bytes,
                  static_cast<hipStream_t>(stream));
}

LMH_API int lmhead_read_n_kept(const void* saved, int64_t* n_kept_host, void* stream) {
  if (!saved || !n_kept_host) return LMHEAD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, saved, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return LMHEAD_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LMHEAD_ERR_HIP;
  *n_kept_host = v;
  return LMHEAD_OK;
}

LMH_API int lmhead_check_status(const void* saved, void* stream) {
  if (!saved) return LMHEAD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SavedHeader h;
  if (hipMemcpyAsync(&h, saved, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess)
    return LMHEAD_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LMHEAD_ERR_HIP;
  return h.status != LMHEAD_OK ? h.status : h.bwd_status;
}

LMH_API const char* lmhead_status_string(int status) {
  switch (status) {
    case LMHEAD_OK: return "ok";
    case LMHEAD_ERR_INVALID_ARG: return "invalid argument";
    case LMHEAD_ERR_UNSUPPORTED: return "unsupported size (H must be a positive multiple of 64)";
    case LMHEAD_ERR_WORKSPACE: return "saved or workspace buffer too small";
    case LMHEAD_ERR_HIP: return "HIP runtime error";
    case LMHEAD_ERR_TARGET_RANGE: return "a kept row's target is outside [0, V)";
    default: return "unknown status";
  }
}

LMH_API int lmhead_version(void) { return kVersion; }

#ifdef LMHEAD_TILE_CLOCKS
// Instrumented builds only (not declared in the public header): copies the
// per-kernel tile clocks (4 kernels x 8 counters, in the order TileClock
// adds them; counter 6 counts workgroups) to host memory after a device
// synchronisation; reset != 0 then zeroes them. Returns 0 or 1 on a HIP error.
LMH_API int lmhead_tile_clocks(unsigned long long* out, int reset) {
  if (!out || hipDeviceSynchronize() != hipSuccess) return 1;
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_tile_clock), sizeof(g_tile_clock)) != hipSuccess)
    return 1;
  if (reset) {
    static const unsigned long long z[4 * 8] = {};
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_tile_clock), z, sizeof(z)) != hipSuccess) return 1;
    if (hipDeviceSynchronize() != hipSuccess) return 1;
  }
  return 0;
}

// out[k][x][0..1]: earliest workgroup start and latest workgroup exit of
// kernel k (fwd, dz, dX, dW) on XCD x, in 100 MHz ticks, since the last reset;
// a reset sets the starts to the largest value and the exits to 0.
LMH_API int lmhead_tile_clocks_xcd(unsigned long long* out, int reset) {
  if (!out || hipDeviceSynchronize() != hipSuccess) return 1;
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_xcd_clock), sizeof(g_xcd_clock)) != hipSuccess)
    return 1;
  if (reset) {
    unsigned long long z[4 * kXcds * 2];
    for (int i = 0; i < 4 * kXcds * 2; ++i) z[i] = (i % 2 == 0) ? ~0ull : 0ull;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_xcd_clock), z, sizeof(z)) != hipSuccess) return 1;
    if (hipDeviceSynchronize() != hipSuccess) return 1;
  }
  return 0;
}
#endif

LMH_API const char* lmhead_kernel_name(int kind) {
  return (kind >= 0 && kind < KK_COUNT) ? kKernelNames[kind] : nullptr;
}

static void prof_release_locked() {
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
}

LMH_API int lmhead_profile_begin(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  prof_release_locked();
  g_prof_on = true;
  return LMHEAD_OK;
}

LMH_API int lmhead_profile_end(double* ms, int64_t* launches) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = false;
  double tot[KK_COUNT] = {0};
  int64_t cnt[KK_COUNT] = {0};
  int st = LMHEAD_OK;
  for (auto& r : g_prof_recs) {
    float e = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&e, r.a, r.b) != hipSuccess) {
      st = LMHEAD_ERR_HIP;
      continue;
    }
    tot[r.kind] += e;
    cnt[r.kind] += 1;
  }
  prof_release_locked();
  for (int k = 0; k < KK_COUNT; ++k) {
    if (ms) ms[k] = tot[k];
    if (launches) launches[k] = cnt[k];
  }
  return st;
}
