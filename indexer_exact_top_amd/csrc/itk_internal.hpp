// Host-side plan structures and launchers shared by the API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/itk.h"

namespace itk {

// Candidate record: the row index and its fp32 value.
struct Cand {
    uint32_t idx;
    float val;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <class T>
struct same_type {
    using type = T;
};

// Launches `kernel` on `stream` and returns the status of this launch only.
// The thread's last-error state is neither read nor cleared, so an error left
// pending by the caller's earlier work stays pending for the caller.
template <class... P>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                typename same_type<P>::type... args)
{
    void *ptrs[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
}

// Planner knobs (process-global, tests only).
struct Knobs {
    int32_t sample_stride = 0;
    float rho = 0.f, rho1 = 0.f;
    int32_t capacity = 0;
    int32_t splits = 0;
    int32_t force_route = 0;
    int32_t route_select = 0;  // ragged mapping: 0 auto, 1 segments, 2 row-local, 3 row-local direct-exact
};
Knobs &knobs();

struct RouteSink {
    int32_t *ptr = nullptr;
    int32_t rows = 0;
    int32_t *count = nullptr;  // admitted candidates per row (fused calls)
    int32_t count_rows = 0;
};
RouteSink &route_sink();

// --------------------------------------------------------------- ragged
constexpr int RAG_THREADS = 256;
constexpr int RAG_WAVES = RAG_THREADS / 64;
// Ragged scan: 16-byte loads per thread per batch (two batches in flight),
// and the longest segment one workgroup scans.
#ifndef RAG_U
#define RAG_U 8
#endif
#ifndef RAG_SEG_MAX
#define RAG_SEG_MAX 32768
#endif
constexpr int RAG_MAX_SPLITS = 64;                      // segments per row chosen by the planner
constexpr int RAG_MAX_CELLS = RAG_MAX_SPLITS * RAG_WAVES; // (segment, wave) cells the finisher gathers on chip
// Ragged finisher: one workgroup per row, 1024 threads for up to 255 rows
// (latency-bound), 512 from 256 rows on (several rows per CU).
constexpr int FIN_THREADS = 1024;
constexpr int FIN_THREADS_MANY = 512;
constexpr int FIN_MANY_ROWS = 256;
// Row-local route: one workgroup of RL_THREADS per row, chunks of RL_U
// 16-byte loads per thread, for at least RAG_RL_MIN_ROWS rows of at most
// RAG_RL_MAX_PITCH scores and secondary counts rho1 * k of at most
// RAG_RL_MAX_CAND (the on-chip stash holds STASH_CAP).  One CU streams a row
// at a few tens of GB/s, so the route needs enough rows to occupy the chip:
// measured on rows of 8K-128K scores (k = 2048), 1024 rows take 76-78 us
// row-local (rows longest first) against 106 us segmented, 64 rows 39 us
// against 22.5 us.
#ifndef RL_THREADS_DEF
#define RL_THREADS_DEF 512
#endif
constexpr int RL_THREADS = RL_THREADS_DEF;
#ifndef RL_U
#define RL_U 4
#endif
constexpr int64_t RAG_RL_MAX_PITCH = 262144;
constexpr int RAG_RL_MIN_ROWS = 512;
constexpr int RAG_RL_MAX_CAND = 4096;
// Row-local direct-exact steps (no view) for rows of at most rho1 * k +
// RAG_DIRECT_MARGIN valid scores: refining an on-chip entry costs about
// 1.3 ns of the workgroup's time and the view about 3.9 us (measured on
// rows of 1K-7.7K scores), so the view pays only when it removes more than
// about 3000 entries.
constexpr int RAG_DIRECT_MARGIN = 3072;
// Row-local stashes for short pitches (a pitch of at most RL_TINY_CAP scores
// takes that stash, else one of at most RL_SMALL_CAP the small one, else
// STASH_CAP).
constexpr int RL_TINY_CAP = 2048;
constexpr int RL_SMALL_CAP = 4096;

struct RaggedPlan {
    int32_t M = 0;
    int64_t pitch = 0;
    int32_t k = 0;
    int32_t P = 1;           // segments per row
    int64_t seg = 0;         // segment length (multiple of 1024)
    int32_t subcap = 0;      // candidate capacity per (segment, wave)
    int32_t bandcap = 0;     // band candidates per row
    int32_t view_blocks = 0; // view stride in 16-element blocks
    float rho = 1.5f, rho1 = 1.75f;
    int32_t force = 0;
    bool rowlocal = false;   // one workgroup per row, candidates on chip
    int32_t rlstash = 0;     // row-local: stash entries of the kernel instance
    int32_t rlcap = 0;       // row-local: on-chip candidate capacity
    uint32_t direct_max = 0; // row-local: rows of at most this length are selected whole (no view)
    // workspace carve
    size_t off_cnt = 0, off_ep = 0, off_slices = 0, off_band = 0, off_order = 0, bytes = 0;
};
RaggedPlan plan_ragged(int32_t M, int64_t pitch, int32_t k);
hipError_t launch_ragged(const RaggedPlan &p, const float *scores, const int32_t *row_len,
                         int32_t *out_idx, void *ws, hipStream_t stream);

// Ragged calls with nothing to refine.  Returns true when the call is
// complete, with its status in *st: a negative size is invalid; no rows or
// k == 0 enqueue nothing; rows of pitch 0 are all empty, so only the -1
// padding of out_idx is written.
bool ragged_trivial(int32_t M, int64_t row_pitch, int32_t k, int32_t *out_idx, hipStream_t stream, itk_status *st);

// ---------------------------------------------------------------- fused
constexpr int FUSED_WAVES = 8;                  // queries per workgroup
constexpr int FUSED_THREADS = FUSED_WAVES * 64;
constexpr int TILE_KEYS = 64;
// Fused select, one workgroup per row: the single-head kernels use 1024
// threads; the head-rows kernel uses 512, because its recovery route holds a
// query's fragments and weights in registers (a 1024-thread workgroup leaves
// 128 VGPRs per lane, which makes it spill).
constexpr int SEL_THREADS = 1024;
constexpr int SEL_THREADS_HR = 512;
constexpr int RESCORE_GROUPS = 256;  // workgroups of the re-scoring kernels (rows are walked)
constexpr int QROW_MAX_SPLITS = 256;  // single-head path: key splits per query
// Head-rows path with at most KP_MAX_T queries: the main pass runs one key
// range per wave, about KP_WAVES waves in all (two per SIMD).  Measured on
// 2^20 FP8 keys, H = 64, D = 128 (main pass): one query 48 us against 72 us
// with the staged scan, two 66 against 79 us; four (104 against 94 us) and
// eight (182 against 145 us) are faster staged, where eight queries share
// each staged key tile.
constexpr int KP_MAX_T = 2;
// Grid-wide recovery passes (head rows): workgroups of FUSED_THREADS, one per CU.
constexpr int RECOVER_WGS = 256;
constexpr int KP_WAVES = 2048;

struct FusedPlan {
    int32_t T = 0, H = 0, D = 0, k = 0;
    int64_t N = 0;
    itk_dtype qt = ITK_BF16, kt = ITK_BF16;
    uint32_t flags = 0;
    int32_t HB = 1;          // 32-head blocks
    int32_t G = 0;           // query groups of FUSED_WAVES
    int32_t P = 1;           // key splits (main pass)
    int32_t Ps = 1;          // key splits (sample passes)
    int64_t span = 0;        // keys per split (multiple of 64), main
    int64_t span_s = 0;      // keys per split, sample
    int32_t sample_tiles = 1;// sampled tile stride
    float rho = 2.0f;
    int32_t cap = 0;         // candidates per row
    int32_t force = 0;
    bool qrow = false;       // single-head path: queries as MFMA columns
    bool kp = false;         // head rows, few queries: main pass with one key range per wave
    int32_t capS = 0;        // single head: candidates per (query, key split)
    int64_t samp_cap = 0;    // single head: stored view scores per query
    size_t off_param = 0, off_mm = 0, off_hist = 0, off_tail = 0, off_gate = 0, off_cand = 0;
    size_t off_hist_r = 0, off_rflag = 0, off_gpub = 0;
    size_t off_samp = 0, off_qcnt = 0, bytes = 0;
    // history sample (head rows only): listed entries, padded entries, key row bytes
    int32_t n_prior = 0, rowb = 0;
    int64_t np = 0;
    size_t off_pidx = 0, off_kp = 0, off_kps = 0, off_pcount = 0;
};
// Largest history sample a fused call takes.
constexpr int32_t PRIOR_MAX = 1 << 16;
itk_status plan_fused(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k, itk_dtype qt, itk_dtype kt,
                      uint32_t flags, FusedPlan *out, int32_t n_prior = 0);
hipError_t launch_fused(const FusedPlan &p, const void *Q, const void *K, const float *k_scale,
                        const float *W, const int32_t *kv_len, int32_t *out_idx, float *out_score,
                        void *ws, hipStream_t stream, const int32_t *prior = nullptr);
// History sample from the previous chunk's lists (count buffer + ragged Top-k).
struct PriorPlan {
    int64_t N = 0;
    int32_t T_prev = 0, k = 0, k_prime = 0, nblk = 0;
    size_t off_count = 0, off_h1 = 0, off_h2 = 0, off_blk = 0, off_par = 0, bytes = 0;
};
itk_status plan_prior(int32_t T_prev, int32_t k, int64_t N, int32_t k_prime, PriorPlan *out);
hipError_t launch_prior(const PriorPlan &p, const int32_t *prev_idx, int32_t *prior_out, void *ws,
                        hipStream_t stream);

// ------------------------------------------------------------ profiling
// Records an event pair around a launch when profiling is enabled.
struct StageTimer {
    int stage;
    hipStream_t stream;
    StageTimer(int stage_id, hipStream_t s);
    ~StageTimer();
};
enum Stage { ST_RAG_SCAN = 0, ST_RAG_FINISH, ST_F_MINMAX, ST_F_HIST, ST_F_MAIN, ST_F_SELECT, ST_RAG_ROWLOCAL, ST_F_RECOVER, ST_F_RESCORE,
             ST_COUNT };

}  // namespace itk
