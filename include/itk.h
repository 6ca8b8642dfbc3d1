/*
 * itk.h — fused Indexer-TopK and exact ragged Top-k for AMD MI355X (gfx950).
 *
 * A small C ABI over hand-written HIP kernels.  Both operations are
 * asynchronous on the caller's HIP stream: they validate their arguments on
 * the host, enqueue a fixed sequence of kernels whose launch geometry depends
 * only on the shape arguments, and return.  They never synchronize, never read
 * device data back to the host and never allocate, so a call can be captured
 * into a HIP graph and replayed.  The caller owns every buffer.
 *
 * Pointers are device pointers unless marked (host).  `stream` is a
 * hipStream_t passed as void* (NULL = the default stream).
 *
 * Error behaviour: an invalid argument is reported synchronously by the status
 * code and nothing is enqueued.  Conditions that depend on device data
 * (too few or too many candidates after the sampled gate, ties, short rows)
 * are never errors: they are resolved on the device by the exact recovery
 * routes, so the result is always the exact Top-k.  Valid lengths larger than
 * the row width are clamped to it; negative lengths are treated as 0.
 */
#ifndef ITK_H
#define ITK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ITK_OK = 0,
    ITK_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad dtype */
    ITK_ERR_UNSUPPORTED = 2,   /* valid but not implemented shape or dtype pair */
    ITK_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    ITK_ERR_HIP = 4,           /* a HIP launch or runtime call failed */
    ITK_ERR_SCRATCH_LIMIT = 5  /* topk_ragged_noalloc: the call needs more than
                                  ITK_RAGGED_NOALLOC_SCRATCH_BYTES of scratch */
} itk_status;

typedef enum {
    ITK_F32 = 0,
    ITK_BF16 = 1,
    ITK_F16 = 2,
    ITK_FP8_E4M3 = 3           /* OCP e4m3fn: 1-4-3, bias 7, max 448, no inf */
} itk_dtype;

/* Flag for indexer_topk_fused: plain inner-product score (k-NN retrieval,
 * LiteTopK Sec. 3.1 Eq. (2)); requires H == 1; W[t,0] still multiplies. */
#define ITK_FLAG_NO_RELU 1u

/* Fused call, FP8 keys only: score with the FP8 matrix cores.  Each
 * (query, head) row of Q is quantized to e4m3fn with its own scale
 * max|Q[t,h,:]| / 448 (round to nearest even), the scale is folded into
 * W[t,h] (exact up to fp32 rounding, since ReLU commutes with a positive
 * factor), and Q8 . K8 runs on v_mfma_scale_f32_32x32x64_f8f6f4.  The scores
 * then approximate the definition by the quantization of Q (the DSA indexer
 * of LiteTopK Sec. 2.1 keeps FP8 keys for this product); the Top-k is exact
 * on those scores.  Requires k_t == ITK_FP8_E4M3, q_t BF16 or F16, H >= 2
 * (ITK_ERR_UNSUPPORTED otherwise). */
#define ITK_FLAG_FP8_SCORE 2u

/* ------------------------------------------------------------------------
 * Standalone exact Top-k over materialized ragged fp32 rows.
 *
 * Operation (Sample-Guided Exact Top-K, arXiv 2609.08450, Sec. 2.1
 * "Operator contract"; exactness criterion Sec. 6.1 Eq. (30)): for each row r
 * with valid length L_r = clamp(row_len[r], 0, row_pitch), return the indices
 * of the min(k, L_r) largest values of scores[r, 0:L_r].  Equal values
 * (including -0 and +0) are resolved in favour of the lower index, so the
 * returned set is unique.  NaN is a precondition violation.
 *
 *   scores   [M, row_pitch] fp32, row-major; only the first L_r entries of a
 *            row are read.  row_pitch % 4 == 0 enables 16-byte loads.
 *   row_len  [M] int32 (device), valid length of each row.
 *   out_idx  [M, k] int32.  The first min(k, L_r) slots of row r hold the
 *            selected indices in unspecified order; the rest hold -1.
 *   workspace / workspace_bytes: scratch of at least
 *            topk_ragged_workspace_size(M, row_pitch, k) bytes, 256-byte
 *            aligned; contents need no initialisation and are meaningless
 *            between calls.  Concurrent calls must not share a workspace.
 *   Empty problems: M == 0 or k == 0 returns ITK_OK with nothing enqueued
 *   and no pointer read; row_pitch == 0 leaves every row empty, so only the
 *   -1 padding of out_idx is written (scores, row_len and the workspace are
 *   not read; the workspace size is 0).  Negative sizes are
 *   ITK_ERR_INVALID_ARG.
 *
 * Method: a block-strided view of the row proposes a coarse boundary, one
 * complete-row pass certifies it and collects the admitted candidates, and an
 * exact radix refinement over (ordered fp32 key, inverted index) resolves the
 * final set; underfilled views fall back to a band pass and then to an exact
 * route that needs no sample (Sec. 4.2-4.4 of the same paper).  A short row
 * (at most 7680 valid entries, the on-chip stash) may instead be refined
 * whole without a view, where the planner finds that faster (the row-local
 * exact mapping of Sec. 5.5).
 * ------------------------------------------------------------------------ */
size_t topk_ragged_workspace_size(int32_t M, int64_t row_pitch, int32_t k);

itk_status topk_ragged(const float *scores, int64_t row_pitch, const int32_t *row_len,
                       int32_t M, int32_t k, int32_t *out_idx,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * topk_ragged without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same operation, arguments, kernels and results as
 * topk_ragged; the scratch comes from a static device array of
 * ITK_RAGGED_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs
 * on holds until the process ends.  The call allocates nothing.
 *
 *   Returns ITK_ERR_SCRATCH_LIMIT, with nothing enqueued, when the shape
 *   needs more scratch than that (topk_ragged_workspace_size(M, row_pitch, k)
 *   gives the need; 64 rows of pitch 131072 with k = 2048 need about 30 MiB).
 *   `stream` must belong to the current device (ITK_ERR_INVALID_ARG
 *   otherwise); NULL is the current device's default stream.
 *   All calls on one GPU share its array: calls that overlap in time on one
 *   GPU (on different streams, or from different threads) race and must be
 *   serialized by the caller.  Each call rewrites the scratch it reads, so
 *   consecutive calls need no clearing.
 * ------------------------------------------------------------------------ */
#define ITK_RAGGED_NOALLOC_SCRATCH_BYTES (64u << 20)

itk_status topk_ragged_noalloc(const float *scores, int64_t row_pitch, const int32_t *row_len,
                               int32_t M, int32_t k, int32_t *out_idx, void *stream);

/* ------------------------------------------------------------------------
 * Fused lightning-indexer score + exact per-row Top-k.
 *
 * Operation (LiteTopK, arXiv 2607.11976, Sec. 2.1 Eq. (1) and Sec. 3.1
 * Eq. (2)): for each query t and each causally valid key j < L_t with
 * L_t = clamp(kv_len[t], 0, N),
 *     s[t,j] = sum_h W[t,h] * ReLU( Q[t,h,:] . Khat[j,:] )
 * (with ITK_FLAG_NO_RELU: s[t,j] = W[t,0] * Q[t,0,:] . Khat[j,:]), where
 * Khat = K for bf16/fp16/fp32 keys and Khat[j,:] = decode(K[j,:]) * k_scale[j]
 * for e4m3fn keys.  Return the min(k, L_t) keys of largest score, ties to the
 * lower index, without materializing the [T, N] score matrix.
 *
 *   Q        [T, H, D] row-major, dtype q_t
 *   K        [N, D] row-major, dtype k_t
 *   k_scale  [N] fp32, required iff k_t == ITK_FP8_E4M3; entries must be
 *            finite and >= 0 (the scale is applied after the ReLU, which is
 *            exact only for non-negative scales).
 *   W        [T, H] fp32 per-query head weights.
 *            Q, K and W must be finite, and the scores must not overflow
 *            fp32: a NaN or infinite score is a precondition violation, as
 *            NaN is for topk_ragged (the result is then unspecified).
 *   kv_len   [T] int32 (device).
 *   out_idx  [T, k] int32: selected key indices in unspecified order, -1 pad.
 *   out_score[T, k] fp32: the kernel's fp32 score of out_idx, -inf pad.
 *   Supported (q_t, k_t): (BF16, BF16), (BF16, FP8_E4M3), (F16, F16),
 *   (F16, FP8_E4M3), (F32, F32).  D in {64, 128, 256}; 1 <= H <= 64;
 *   H > 32 needs D <= 128; F32 needs ceil(H/32) * D <= 128.
 *   Scores are accumulated in fp32 (MFMA); selection is exact on those fp32
 *   scores.  Scratch is O(T * k): see the workspace size query.
 *   With H == 1 and 16-bit inputs the scores come from a separate kernel
 *   family (queries as MFMA columns, 512 per workgroup); its workspace also
 *   holds every query's sampled-view scores (at most about 32768 per query).
 *   Results follow the same contract on either path.
 *   workspace: as for topk_ragged.
 *   Empty problems: once H, D, the dtypes and the flags pass the checks of
 *   a non-empty call, T == 0 or k == 0 returns ITK_OK with nothing enqueued
 *   and no pointer read; N == 0 leaves every row empty, so only the padding
 *   of out_idx and out_score is written (Q, K, k_scale, W, kv_len and the
 *   workspace are not read; the workspace size is 0).  Negative sizes are
 *   ITK_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
size_t indexer_topk_fused_workspace_size(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k,
                                         itk_dtype q_t, itk_dtype k_t, uint32_t flags);

itk_status indexer_topk_fused(const void *Q, itk_dtype q_t, const void *K, itk_dtype k_t,
                              const float *k_scale, const float *W, const int32_t *kv_len,
                              int32_t T, int32_t H, int32_t D, int64_t N, int32_t k,
                              uint32_t flags, int32_t *out_idx, float *out_score,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Fused call with a history sample.
 *
 * Same operation, arguments and result as indexer_topk_fused; the initial
 * gate comes from a caller-given list of keys instead of the strided view
 * (LiteTopK, arXiv 2607.11976, Sec. 3.2 "Sampling"): the keys of the previous
 * chunk's Top-k lists that occur most often (indexer_prior_from_topk below
 * makes that list; about 3k entries for sparse attention).  Every query
 * scores the listed keys below its own length; since they are keys of its
 * own row, the k-th largest of their scores cannot exceed the row's k-th
 * largest, and the gate is placed at the bin holding it, so every key of the
 * Top-k passes.
 *
 *   prior_idx  [n_prior] int32 (device) key indices, any order.  Entries
 *              outside [0, N) are ignored; a key listed twice is scored twice
 *              and weakens the gate's guarantee, never the result.
 *   n_prior    0 <= n_prior <= 65536; 0 gives the strided view, as
 *              indexer_topk_fused does.  A query with fewer than k listed
 *              keys below its length gets no gate (all its keys are
 *              candidates, resolved by the recovery passes).
 *   Rejected with ITK_ERR_UNSUPPORTED on the single-head path (H == 1 with
 *   16-bit Q): LiteTopK keeps the history sample for sparse attention and
 *   samples k-NN rows, which have no such temporal structure.
 *   The workspace size depends on n_prior.
 * ------------------------------------------------------------------------ */
size_t indexer_topk_fused_prior_workspace_size(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k,
                                               itk_dtype q_t, itk_dtype k_t, uint32_t flags, int32_t n_prior);

itk_status indexer_topk_fused_prior(const void *Q, itk_dtype q_t, const void *K, itk_dtype k_t,
                                    const float *k_scale, const float *W, const int32_t *kv_len,
                                    int32_t T, int32_t H, int32_t D, int64_t N, int32_t k, uint32_t flags,
                                    const int32_t *prior_idx, int32_t n_prior,
                                    int32_t *out_idx, float *out_score,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* The history sample of the next chunk (LiteTopK Sec. 3.2 "Sampling"): the
 * k_prime keys that occur most often in the previous chunk's lists.
 *
 *   prev_idx   [T_prev, k] int32 (device): the previous chunk's out_idx.
 *              Entries outside [0, N) (the -1 padding) count for nothing.
 *   prior_out  [k_prime] int32: of the keys sorted by (count descending,
 *              index ascending), the first min(k_prime, N), written in
 *              ascending index order; slots past min(k_prime, N) hold -1.
 *   Requires T_prev * k < 2^25 (ITK_ERR_UNSUPPORTED otherwise), T_prev >= 0,
 *   k > 0, 0 < N <= 2^31 - 1, k_prime > 0.
 *   Scratch: indexer_prior_workspace_size bytes (4 N plus about 50 KB).
 *   Can run on its own stream, beside the current chunk's work.
 */
size_t indexer_prior_workspace_size(int32_t T_prev, int32_t k, int64_t N, int32_t k_prime);

itk_status indexer_prior_from_topk(const int32_t *prev_idx, int32_t T_prev, int32_t k, int64_t N,
                                   int32_t k_prime, int32_t *prior_out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *itk_status_string(itk_status status);

/* Name of the HIP runtime error behind the calling thread's most recent
 * ITK_ERR_HIP ("hipSuccess" if there was none; static storage). */
const char *itk_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Test and measurement knobs (not needed for normal use).
 * ------------------------------------------------------------------------ */

/* Planner overrides.  A zero field keeps the default.  Process-global; they
 * change efficiency, never results.  Workspace sizes depend on `capacity`,
 * so query the size after setting the knobs. */
typedef struct {
    int32_t sample_stride;  /* ragged: view density 1/s (one 16-element block in s);
                               fused: sampled tile stride (1 in N tiles of 64 keys) */
    float rho;              /* primary target rank as a multiple of k */
    float rho1;             /* ragged: secondary (band) target rank multiple */
    int32_t capacity;       /* fused: candidates per row; ragged: per segment */
    int32_t splits;         /* fused: key splits per query group;
                               ragged: segments per row */
    int32_t force_route;    /* 0 auto; 1 exact route for every row (ragged:
                               no sample; fused: re-scoring recovery);
                               2 ragged: force the band pass */
    int32_t ragged_route;   /* ragged mapping: 0 auto (by shape), 1 segments
                               (view + scan per segment, finish per row),
                               2 row-local (one workgroup per row, sampled
                               steps for every row), 3 row-local with the
                               direct-exact steps (no view) for every row of
                               at most 7680 valid scores (or `capacity`);
                               row-local is taken only for rows of at most
                               262144 scores and rho1 * k <= 4096, or a
                               pitch of at most 7680 */
} itk_plan_opts;

/* NULL restores the defaults. */
itk_status itk_set_plan_opts(const itk_plan_opts *opts);

/* Route taken per row by the last calls: when `route_out` (device, [rows]
 * int32) is non-NULL, each following call writes a route code per row:
 *   1 certified by the sample, 2 certified after the band pass,
 *   3 exact route (no usable sample, overflow, or underfill; for fused calls
 *     the single-workgroup re-scoring that remains when a row's boundary bin
 *     alone overflows the buffer),
 *   4 all valid entries fit the candidate capacity (no gate needed),
 *   5 fused calls: recovered by the grid-wide recovery passes (overflow or
 *     underfill of the sampled gate).
 * Pass NULL to stop. */
itk_status itk_set_route_buffer(int32_t *route_out, int32_t rows);

/* Candidates per row: when `count_out` (device, [rows] int32) is non-NULL,
 * each following fused call writes, per query row, the number of candidates
 * its selection started from (admitted by the gate of the main pass, or
 * collected by the recovery passes for a recovered row; the single-head path
 * counts every admitted key, also past the slices' capacity).  Pass NULL to
 * stop. */
itk_status itk_set_count_buffer(int32_t *count_out, int32_t rows);

/* Per-kernel timing.  While enabled, each call records HIP events around each
 * kernel it launches; itk_profile_read sums the elapsed milliseconds per
 * stage since the last read (synchronizing on the recorded events) and
 * returns the number of stages written.  Stage names are static strings. */
itk_status itk_profile_enable(int32_t on);
int32_t itk_profile_read(double *ms_out, int32_t *count_out, const char **names_out, int32_t max_stages);

#ifdef __cplusplus
}
#endif

#endif /* ITK_H */
