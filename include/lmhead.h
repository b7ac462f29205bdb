/*
 * lmhead.h - C ABI of the fused LM-head log-prob / entropy op for MI355X (gfx950).
 *
 * The op takes final hidden states X [N, H] and the vocabulary weight W [V, H]
 * (both bf16, row-major) and returns, per token, the log-probability of its
 * target token and the entropy of its next-token distribution, plus the
 * backward pass into dX and dW, without ever writing the [N, V] logits to
 * memory.
 *
 * Sources (all behaviour below is defined by these pages):
 *  - prime-rl PR #3326, "Don't compute the logprobs and their gradients for
 *    tokens no loss com...": author comment (the vocab matmul is where the
 *    FLOPs are; tokens no loss reads are skipped) and Overview (a keep mask
 *    selects positions; compact -> chunked log-prob/entropy -> expand back,
 *    with zero log-prob and entropy at skipped positions; the token chunk
 *    bounds memory).
 *  - SkyRL PR #2374, "feat(megatron): fuse LM-head entropy for RL": "How it
 *    works" and "Usage" (one projection gives selected-token log-probs and
 *    entropy; metric-only entropy adds no gradient work; entropy-loss mode
 *    keeps the entropy derivative; the caller's gradient requirement selects
 *    it), and the gemini-code-assist review (entropy saved for backward, not
 *    recomputed).
 *  - twinkle PR #283, "Fix three memory defects in the Megatron path",
 *    section 1 (float32 compute; float32 log-probs and entropies for bf16
 *    inputs; the softmax is recomputed in backward from saved inputs, never
 *    stored).
 *
 * Definitions, per kept row i with z = W x_i (fp32 accumulation of bf16
 * products) and LSE_i = log sum_v exp(z_v):
 *   logp_i    = z_{t_i} - LSE_i
 *   entropy_i = -sum_v p_v log p_v,   p_v = exp(z_v - LSE_i)   (nats)
 * Skipped rows (keep_mask[i] == 0) get logp = +0.0 and entropy = +0.0, their
 * dX row is +0.0 and they contribute nothing to dW.
 * Backward, for the loss L = sum_i g_lp[i] logp_i + [entropy_requires_grad]
 * g_H[i] entropy_i:
 *   dZ_i = g_lp[i] (onehot(t_i) - p) - [entropy_requires_grad] g_H[i] p (log p + entropy_i)
 *   dX_i = dZ_i W          dW = sum_i dZ_i^T x_i
 * dZ is rounded to bf16 (round to nearest even) before the two products.
 *
 * Conventions
 *  - Every tensor pointer is a DEVICE pointer, caller-owned, 16-byte aligned
 *    (256-byte alignment recommended). The library never allocates device
 *    memory and never synchronises, except in the two calls marked "syncs".
 *  - All work is enqueued on `stream` (a hipStream_t; 0 = the null stream)
 *    in stream order. Calls are reentrant and keep no state between calls
 *    other than a per-device cache of the compute-unit count.
 *  - Every call returns an lmhead_status. All argument checks run on the host
 *    before anything is enqueued; a failing call enqueues nothing.
 *  - Sizes: N >= 0, V >= 1, H >= 64 with H % 64 == 0 (else
 *    LMHEAD_ERR_UNSUPPORTED). N and V are otherwise arbitrary up to
 *    N <= 2^24, V <= 2^22, H <= 2^20 (else LMHEAD_ERR_UNSUPPORTED): within
 *    them every matrix the kernels read is addressed through 32-bit buffer
 *    offsets that stay below 2^31 bytes, and every tile index fits int32.
 *  - Results are bitwise reproducible run to run for the same inputs and
 *    arguments (fixed reduction orders, no floating-point atomics).
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMHEAD_OK = 0,
  LMHEAD_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, bad flag combination, misalignment */
  LMHEAD_ERR_UNSUPPORTED = 2,   /* H % 64 != 0 or H < 64, sizes beyond int32 indexing */
  LMHEAD_ERR_WORKSPACE = 3,     /* saved or workspace buffer smaller than the size query returns */
  LMHEAD_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  LMHEAD_ERR_TARGET_RANGE = 5   /* a kept row's target is outside [0, V) */
} lmhead_status;

/* Bytes of the `saved` buffer lmhead_fwd fills for lmhead_bwd: a small header,
 * the ascending kept-row positions, a per-row position map, and per kept row
 * the log-sum-exp and the entropy (16 bytes per row plus 1 KiB). The saved
 * state never holds a full-vocabulary activation (twinkle PR #283, section 1).
 * Returns 0 if N < 0. */
size_t lmhead_saved_bytes(int64_t N);

/* Workspace bytes lmhead_fwd needs for N rows and vocabulary V: 8 tile-queue
 * counters, the target of each kept row (N rounded up to 256 entries), per
 * row the target logit and, per 256-wide vocabulary tile, three fp32 partial
 * statistics, plus a bf16 transposed copy of the kept rows of X
 * ([H][N rounded up to 64]). Returns 0 on invalid sizes. */
size_t lmhead_fwd_workspace_bytes(int64_t N, int64_t H, int64_t V);

/* Workspace bytes lmhead_bwd needs: a 256-byte checked copy of the saved
 * header, 32 tile-queue counters per token chunk, 20 bytes per kept row (N
 * rounded up to 256 entries) of logit-gradient coefficients and targets, a
 * bf16 transposed copy of one chunk's kept rows of X ([H][C + 64]), the bf16
 * logit gradient dZ of one chunk of C rows ([C][V rounded up to 256, + 64],
 * token-major; the 64 padding elements of a row keep power-of-two row pitches
 * out of these two buffers), where C = token_chunk rounded up to a multiple
 * of 256, at most N rounded up
 * to 256 and at most 2^22 (a larger request is clamped to 2^22), and, for
 * V >= 2048, fp32 partial dX tiles: when the dX tiles of a chunk past its
 * last whole round of workgroups number at most 256 (S - 1) / S, each is
 * computed as S pieces of the vocabulary range that the whole device runs,
 * then summed in a fixed order; S = 8 when 8 pieces of a multiple of 64
 * vocabulary rows fit in V rounded up to 256, else 4
 * (min(256 (S - 1) / S, C / 256 * ceil(H / 256)) * S tiles of 256 x 256).
 * token_chunk <= 0 selects the largest chunk whose dZ fits 8 GiB (prime-rl PR
 * #3326, Overview, uses the chunk to bound memory; its default of 8192 rows
 * was set for a smaller memory). Returns 0 on invalid sizes. */
size_t lmhead_bwd_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t token_chunk);

/* Forward: compaction of the kept rows, the fused projection with per-row
 * online max / sum-exp / sum p*z statistics over vocabulary tiles, the
 * target-logit pick, the fixed-order merge, and the expand-back.
 *
 *  hidden     bf16 [N, H] row-major
 *  weight     bf16 [V, H] row-major
 *  targets    int32 [N]; only kept rows are read. A kept target outside
 *             [0, V) yields logp = NaN at that row and is reported by
 *             lmhead_check_status.
 *  keep_mask  uint8 [N], nonzero = keep; NULL = keep every row
 *  logp       fp32 [N] out, fully written (+0.0 at skipped rows)
 *  entropy    fp32 [N] out, fully written; must be NULL iff !return_entropy
 *             (not checked when N == 0, where any output may be NULL)
 *  entropy_requires_grad  requires return_entropy (else INVALID_ARG); it is
 *             recorded in `saved`, and lmhead_bwd must pass the same value.
 *  saved      device buffer of >= lmhead_saved_bytes(N) bytes, out
 *  workspace  device buffer of >= lmhead_fwd_workspace_bytes(N, H, V) bytes;
 *             free for reuse once the enqueued work has completed.
 *  N == 0 is valid and enqueues a header write only.
 */
int lmhead_fwd(const void* hidden, const void* weight, const int32_t* targets,
               const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
               int return_entropy, int entropy_requires_grad,
               float* logp, float* entropy,
               void* saved, size_t saved_bytes,
               void* workspace, size_t workspace_bytes,
               void* stream);

/* Block-sparse forward: the same arguments, outputs and saved state as
 * lmhead_fwd, but rows are not compacted. The rows are taken in place in
 * tiles of 256 consecutive rows (the GEMMs' token tile), and only tiles with
 * no kept row are skipped (SkyRL PR #2374, "How it works": block-sparse
 * forward and backward that skip inactive tiles). Every row of a tile that
 * holds a kept row runs through the projection. Rows that are not kept still
 * get +0.0 log-prob and entropy, and lmhead_bwd gives them an all-zero logit
 * gradient: a +0.0 dX row and no dW contribution. Per row, log-prob and
 * entropy equal those of lmhead_fwd bit for bit, because a row's results do
 * not depend on which other rows share its tile; so does dX unless the two
 * row counts split the dX tail differently (see lmhead_bwd_workspace_bytes),
 * when it agrees to rounding. dW sums the same rows with zero rows between
 * them, in a different order, so it agrees to rounding. The saved header counts the listed rows as n_kept (what
 * lmhead_read_n_kept reports) and sets bit 2 of its flags. Take the
 * backward with lmhead_bwd. Same errors as lmhead_fwd. */
int lmhead_fwd_blocksparse(const void* hidden, const void* weight, const int32_t* targets,
                           const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
                           int return_entropy, int entropy_requires_grad,
                           float* logp, float* entropy,
                           void* saved, size_t saved_bytes,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). It is lmhead_fwd with its workspace in a device array built
 * into the library: LMHEAD_NOALLOC_SCRATCH_BYTES bytes on each GPU the
 * library runs on, held until the process ends. The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine, no timing events
 * while lmhead_profile_begin is on). Same arguments, outputs and saved state
 * as lmhead_fwd, without the workspace; the backward is lmhead_bwd.
 *  Errors: as lmhead_fwd, plus LMHEAD_ERR_WORKSPACE when
 *  lmhead_fwd_workspace_bytes(N, H, V) exceeds LMHEAD_NOALLOC_SCRATCH_BYTES
 *  (e.g. N 8192, H 4096, V 131072 fits; N 16384 at that H and V does not),
 *  and LMHEAD_ERR_HIP if the array's device address cannot be obtained.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (each call rewrites what it reads). Calls that overlap on one GPU
 * -- on different streams, or from host threads whose work is not ordered
 * on one stream -- race; calls in one stream's order do not.
 */
#define LMHEAD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int lmhead_fwd_noalloc(const void* hidden, const void* weight, const int32_t* targets,
                       const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V,
                       int return_entropy, int entropy_requires_grad,
                       float* logp, float* entropy,
                       void* saved, size_t saved_bytes,
                       void* stream);

/* Backward: per chunk of `token_chunk` kept rows, recompute the logit tile,
 * form dZ (above) in bf16, then dX rows = dZ W (scattered back to the rows'
 * original positions) and dW (+)= dZ^T X. The first chunk writes dW, later
 * chunks add to it in ascending chunk order.
 *
 *  hidden, weight, targets, N, H, V: exactly as passed to lmhead_fwd
 *  entropy_requires_grad: as passed to lmhead_fwd
 *  saved      the buffer lmhead_fwd filled. Its header records the forward's
 *             N, H, V and entropy_requires_grad; the backward compares them
 *             with its own arguments on the device (it cannot read them
 *             without synchronising). On a mismatch it computes nothing from
 *             the saved state: grad_hidden and grad_weight are written with
 *             +0.0 everywhere, and lmhead_check_status(saved) then returns
 *             LMHEAD_ERR_INVALID_ARG. The backward writes one word of `saved`,
 *             the check's result (LMHEAD_OK for a consistent call), and nothing else.
 *  grad_logp  fp32 [N]; skipped rows are not read
 *  grad_entropy fp32 [N]; must be NULL iff !entropy_requires_grad (N > 0)
 *  grad_hidden fp32 [N, H] out, fully overwritten (+0.0 rows where skipped)
 *  grad_weight fp32 [V, H] out, fully overwritten
 *  token_chunk rows per chunk, rounded up to a multiple of 256; <= 0 selects
 *             the default described at lmhead_bwd_workspace_bytes
 *  workspace  >= lmhead_bwd_workspace_bytes(N, H, V, token_chunk) bytes
 */
int lmhead_bwd(const void* hidden, const void* weight, const int32_t* targets,
               int64_t N, int64_t H, int64_t V, int entropy_requires_grad,
               const void* saved, size_t saved_bytes,
               const float* grad_logp, const float* grad_entropy,
               float* grad_hidden, float* grad_weight,
               int64_t token_chunk, void* workspace, size_t workspace_bytes,
               void* stream);

/* Vocabulary-shard forward. The weight rows of a vocabulary of V_total
 * entries are split over several calls (one per rank under tensor
 * parallelism); this call reads the shard of rows [vocab_start, vocab_start +
 * V_shard) and writes, per row, its statistics over the shard. In SkyRL PR
 * #2374 each rank reduces over its vocabulary shard and the ranks combine the
 * results with collectives over the tensor-parallel group (gemini-code-assist
 * review); here the per-row combine is lmhead_merge_partials, so one
 * all-gather of these 16-byte records is the only exchange the forward needs.
 *
 *  hidden, targets, keep_mask, N, H: as for lmhead_fwd; targets are indices
 *             into the whole vocabulary [0, V_total)
 *  weight_shard bf16 [V_shard, H] row-major: rows vocab_start .. of the weight
 *  partial    fp32 [N, 4] out: {m, s, b, z_t} per row, natural-log units,
 *             m = max z, s = sum e^(z - m), b = sum e^(z - m) (z - m) over the
 *             shard's logits z; z_t = the target logit if the target lies in
 *             the shard, else NaN. Skipped rows: {-inf, 0, 0, NaN}.
 *  saved      >= lmhead_saved_bytes(N) bytes, out: compaction state; every
 *             shard's call fills an identical copy, and lmhead_merge_partials
 *             completes it (LSE, entropy) for lmhead_bwd_partial
 *  workspace  >= lmhead_fwd_workspace_bytes(N, H, V_shard) bytes
 *  Requires 0 <= vocab_start, vocab_start + V_shard <= V_total <= 2^22. A
 *  kept target outside [0, V_total) is reported by lmhead_check_status.
 */
int lmhead_fwd_partial(const void* hidden, const void* weight_shard, const int32_t* targets,
                       const uint8_t* keep_mask, int64_t N, int64_t H, int64_t V_shard,
                       int64_t vocab_start, int64_t V_total, float* partial,
                       void* saved, size_t saved_bytes,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Combines the records of P vocabulary shards that together cover the
 * vocabulary (disjoint ranges, any order of ranges, combined in the order
 * given) into the full op's outputs: LSE = m + ln s and entropy = ln s - b / s
 * of the merged statistics, log-prob = z_t - LSE with z_t from the one shard
 * that holds the target (NaN if none does).
 *
 *  partials   fp32 [P, N, 4]: the P shards' records, each as lmhead_fwd_partial
 *             wrote it
 *  logp       fp32 [N] out (+0.0 at skipped rows)
 *  entropy    fp32 [N] out; must be NULL iff !return_entropy (N > 0)
 *  entropy_requires_grad  requires return_entropy; recorded in `saved`
 *  saved      a buffer lmhead_fwd_partial filled for these rows; its LSE and
 *             entropy are written here
 */
int lmhead_merge_partials(const float* partials, int64_t P, int64_t N,
                          int return_entropy, int entropy_requires_grad,
                          float* logp, float* entropy,
                          void* saved, size_t saved_bytes, void* stream);

/* Vocabulary-shard backward: lmhead_bwd restricted to the shard's logits,
 * with the LSE and entropy of the whole vocabulary from `saved` (after
 * lmhead_merge_partials). grad_hidden is this shard's share dZ_shard W_shard of
 * dX: the caller sums it over the shards (one all-reduce), as SkyRL PR #2374
 * leaves the hidden-gradient reduction to the caller (cursor and greptile
 * reviews); grad_weight_shard is exactly the shard's rows of dW.
 *
 *  hidden, targets, N, H, entropy_requires_grad, grad_logp, grad_entropy,
 *             token_chunk: as for lmhead_bwd
 *  weight_shard, V_shard, vocab_start: as passed to lmhead_fwd_partial
 *  saved      completed by lmhead_merge_partials (its entropy_requires_grad
 *             is the one this call must pass); checked as in lmhead_bwd, with
 *             the shard's range required to lie inside the forward's
 *             vocabulary. A state that lmhead_merge_partials never completed
 *             is rejected the same way (+0.0 gradients, INVALID_ARG status).
 *  grad_hidden fp32 [N, H] out, fully overwritten (+0.0 rows where skipped)
 *  grad_weight_shard fp32 [V_shard, H] out, fully overwritten
 *  workspace  >= lmhead_bwd_workspace_bytes(N, H, V_shard, token_chunk) bytes
 */
int lmhead_bwd_partial(const void* hidden, const void* weight_shard, const int32_t* targets,
                       int64_t N, int64_t H, int64_t V_shard, int64_t vocab_start,
                       int entropy_requires_grad, const void* saved, size_t saved_bytes,
                       const float* grad_logp, const float* grad_entropy,
                       float* grad_hidden, float* grad_weight_shard,
                       int64_t token_chunk, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Logits that already exist: log-prob and entropy from a caller-held
 * [N, V] logit matrix, the selective_log_softmax contract of twinkle PR #283,
 * section 1 (fp32 results for bf16 logits; the backward recomputes the
 * softmax from the logits instead of keeping it). One pass over each row in
 * each direction and no temporaries, so the pages' row chunking, which bounds
 * temporaries, is not needed. A -inf logit counts as probability 0.
 */
#define LMHEAD_DTYPE_BF16 0
#define LMHEAD_DTYPE_F32 1

/*  logits     [N, V] row-major, dtype LMHEAD_DTYPE_BF16 (2-byte aligned) or
 *             LMHEAD_DTYPE_F32 (4-byte aligned); any V >= 1
 *  targets    int32 [N]; a kept target outside [0, V) gives logp = NaN
 *  keep_mask  uint8 [N] (nonzero = keep) or NULL; skipped rows get +0.0
 *  logp       fp32 [N] out; entropy fp32 [N] out, NULL iff !return_entropy
 *  saved_stats fp32 [N, 2] out: {LSE, entropy} per row (0 for skipped rows),
 *             the state lmhead_logits_bwd needs
 */
int lmhead_logits_fwd(const void* logits, int dtype, int64_t N, int64_t V,
                      const int32_t* targets, const uint8_t* keep_mask,
                      int return_entropy, float* logp, float* entropy,
                      float* saved_stats, void* stream);

/* dL/dlogits = g_lp (onehot(t) - p) - g_H p (ln p + H), p = softmax(row),
 * the entropy term only if entropy_requires_grad; written in the logits'
 * dtype (bf16 rounds to nearest even), +0.0 rows where skipped.
 *
 *  logits, dtype, N, V, targets, keep_mask: as passed to lmhead_logits_fwd
 *  saved_stats  as lmhead_logits_fwd wrote it
 *  grad_logp    fp32 [N]; grad_entropy fp32 [N], NULL iff !entropy_requires_grad
 *  grad_logits  [N, V] out in `dtype`, fully overwritten; its address must
 *               have the same offset modulo 16 bytes as `logits`
 */
int lmhead_logits_bwd(const void* logits, int dtype, int64_t N, int64_t V,
                      const int32_t* targets, const uint8_t* keep_mask,
                      const float* saved_stats, const float* grad_logp,
                      const float* grad_entropy, int entropy_requires_grad,
                      void* grad_logits, void* stream);

/* Syncs `stream`, then reads the number of kept rows from `saved` into
 * *n_kept_host (the token fraction the trainer logs, prime-rl PR #3326,
 * Overview); after lmhead_fwd_blocksparse, the number of rows in the tiles it
 * ran. */
int lmhead_read_n_kept(const void* saved, int64_t* n_kept_host, void* stream);

/* Syncs `stream`, then returns LMHEAD_ERR_TARGET_RANGE if the forward that
 * filled `saved` met a kept row whose target is outside [0, V); else
 * LMHEAD_ERR_INVALID_ARG if the last backward on `saved` found it
 * inconsistent with its arguments (see lmhead_bwd); else LMHEAD_OK. */
int lmhead_check_status(const void* saved, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* lmhead_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int lmhead_version(void);

/* Per-kernel timing for benchmarks (not needed to use the op).
 * Kernel kinds, in order: compact, gather_cols, fwd_tiles, merge,
 * zero_skipped, zero_rows, dz_tiles, dx_tiles, dw_tiles, zero_queues,
 * bwd_rows, merge_shards, dx_reduce, dxdw_tiles (dX's whole tiles and then
 * dW in one launch; dx_tiles is then the split tail's pieces, dw_tiles a dW
 * launch of a batch with no rows). */
#define LMHEAD_NUM_KERNELS 14

/* Static name of kernel kind `kind` (NULL if out of range). */
const char* lmhead_kernel_name(int kind);

/* While profiling is on, every launch the library makes (from any host thread,
 * on any stream) is bracketed by a hipEvent pair recorded on the launch
 * stream. lmhead_profile_begin clears previous records; it creates events but
 * allocates no device memory. */
int lmhead_profile_begin(void);

/* Stops recording, waits for the recorded events, and writes per-kind totals:
 * ms[k] = summed event time of kind k's launches, launches[k] = their count
 * (arrays of LMHEAD_NUM_KERNELS; either may be NULL). Syncs the events. */
int lmhead_profile_end(double* ms, int64_t* launches);

/* MFMA ceiling probe for benchmarks (not needed to use the op).
 * Runs the GEMM kernels' inner step -- v_mfma_f32_16x16x32_bf16 in 8 x 8
 * blocks per wave, in the engine's order, four waves per workgroup, one
 * workgroup per CU -- with all operands in registers: no loads, no LDS
 * traffic, no barriers. `iters` passes of two k steps each; the flop count is
 * exact. Its rate bounds what the GEMM
 * kernels can reach at the clock the chip holds under MFMA load, which
 * depends on how often operand bits switch: operand fragments are read once
 * from `a` and `b` (device bf16 arrays of a_elems / b_elems >= 8 entries,
 * 16-byte aligned; pass the GEMMs' own operands to get their bit statistics),
 * or are all zero when both are NULL.
 *   workspace: device, 16-byte aligned, >= lmhead_mfma_probe_workspace_bytes()
 *     (per-workgroup cycle counts and a per-thread sum that keeps the products
 *     live; overwritten).
 *   ms: elapsed kernel time (hipEvents on `stream`); flops: work done;
 *   clock_ghz: mean s_memtime cycles of a workgroup's loop / elapsed time.
 * Any output pointer may be NULL. Syncs `stream`. Errors: INVALID_ARG for
 * iters outside [1, 2^24], one of a / b NULL, a short or misaligned array;
 * WORKSPACE for a small workspace; HIP for a failed launch or event. */
size_t lmhead_mfma_probe_workspace_bytes(void);
int lmhead_mfma_probe(const void* a, int64_t a_elems, const void* b, int64_t b_elems,
                      int64_t iters, void* workspace, size_t workspace_bytes,
                      double* ms, double* flops, double* clock_ghz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
