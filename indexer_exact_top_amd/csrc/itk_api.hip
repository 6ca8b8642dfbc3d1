// C ABI: argument validation, planning, workspace carving and launches.
// Nothing here reads device data or allocates device memory.
#include <math.h>
#include <mutex>
#include <vector>

#include "fused_qrow.hpp"
#include "itk_internal.hpp"

namespace itk {

Knobs &knobs()
{
    static Knobs k;
    return k;
}

RouteSink &route_sink()
{
    static RouteSink r;
    return r;
}

FusedLauncher find_fused_launcher_bf16(int, int, int, int, bool, bool);
FusedLauncher find_fused_launcher_f16(int, int, int, int, bool, bool);
FusedLauncher find_fused_launcher_f32(int, int, int, int, bool, bool);

FusedLauncher find_qrow_launcher_bf16(int, int, int, bool);
FusedLauncher find_qrow_launcher_f16(int, int, int, bool);

FusedLauncher find_qrow_launcher(int qt, int kt, int d, bool relu)
{
    if (qt == ITK_BF16) return find_qrow_launcher_bf16(qt, kt, d, relu);
    if (qt == ITK_F16) return find_qrow_launcher_f16(qt, kt, d, relu);
    return nullptr;
}

FusedLauncher find_fused_launcher(int qt, int kt, int hb, int d, bool relu, bool q8)
{
    if (qt == ITK_BF16) return find_fused_launcher_bf16(qt, kt, hb, d, relu, q8);
    if (qt == ITK_F16) return find_fused_launcher_f16(qt, kt, hb, d, relu, q8);
    if (qt == ITK_F32) return find_fused_launcher_f32(qt, kt, hb, d, relu, q8);
    return nullptr;
}

// ---------------------------------------------------------- profiling
namespace {
struct ProfRec {
    int stage;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
const char *const g_stage_names[ST_COUNT] = {"ragged_scan",      "ragged_finish", "fused_sample_range",
                                             "fused_sample_hist", "fused_main",    "fused_select",
                                             "ragged_rowlocal", "fused_recover",    "fused_rescore"};
}  // namespace

StageTimer::StageTimer(int stage_id, hipStream_t s) : stage(-1), stream(s)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    ProfRec r{stage_id, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess) return;
    if (hipEventCreate(&r.b) != hipSuccess) {
        (void)hipEventDestroy(r.a);
        return;
    }
    (void)hipEventRecord(r.a, stream);
    g_prof.push_back(r);
    stage = stage_id;
}

StageTimer::~StageTimer()
{
    if (stage < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    (void)hipEventRecord(g_prof.back().b, stream);
}

static uint64_t ceil_div_u(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

itk_status plan_fused(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k, itk_dtype qt, itk_dtype kt,
                      uint32_t flags, FusedPlan *out, int32_t n_prior)
{
    if (T <= 0 || H <= 0 || D <= 0 || N <= 0 || k <= 0 || n_prior < 0) return ITK_ERR_INVALID_ARG;
    if (n_prior > PRIOR_MAX) return ITK_ERR_UNSUPPORTED;
    if (N > (int64_t)0x7FFFFFFF) return ITK_ERR_UNSUPPORTED;
    if (qt < ITK_F32 || qt > ITK_FP8_E4M3 || kt < ITK_F32 || kt > ITK_FP8_E4M3) return ITK_ERR_INVALID_ARG;
    if (flags & ~(ITK_FLAG_NO_RELU | ITK_FLAG_FP8_SCORE)) return ITK_ERR_INVALID_ARG;
    if ((flags & ITK_FLAG_NO_RELU) && H != 1) return ITK_ERR_INVALID_ARG;
    const bool q8 = (flags & ITK_FLAG_FP8_SCORE) != 0;
    if (q8 && (kt != ITK_FP8_E4M3 || qt == ITK_F32 || H < 2)) return ITK_ERR_UNSUPPORTED;
    if (H > 64) return ITK_ERR_UNSUPPORTED;
    if (D != 64 && D != 128 && D != 256) return ITK_ERR_UNSUPPORTED;
    const bool pair_ok = (qt == ITK_BF16 && (kt == ITK_BF16 || kt == ITK_FP8_E4M3)) ||
                         (qt == ITK_F16 && (kt == ITK_F16 || kt == ITK_FP8_E4M3)) ||
                         (qt == ITK_F32 && kt == ITK_F32);
    if (!pair_ok) return ITK_ERR_UNSUPPORTED;
    const int HB = (H + 31) / 32;
    if (HB == 2 && D > 128) return ITK_ERR_UNSUPPORTED;
    if (qt == ITK_F32 && HB * D > 128) return ITK_ERR_UNSUPPORTED;
    const bool relu = !(flags & ITK_FLAG_NO_RELU);
    if (!find_fused_launcher(qt, kt, HB, D, relu, q8)) return ITK_ERR_UNSUPPORTED;

    const Knobs &kn = knobs();
    FusedPlan p;
    p.T = T; p.H = H; p.D = D; p.N = N; p.k = k; p.qt = qt; p.kt = kt; p.flags = flags; p.HB = HB;
    if (H == 1 && qt != ITK_F32 && find_qrow_launcher(qt, kt, D, relu)) {
        // no history sample here: LiteTopK Sec. 3.2 keeps the history sample
        // for sparse attention and samples k-NN rows, which carry no such
        // temporal structure
        if (n_prior > 0) return ITK_ERR_UNSUPPORTED;
        // Single head: queries are the MFMA columns (32 per block, QROW_Q per
        // workgroup); keys are split so that about 256 workgroups run.
        p.qrow = true;
        p.G = (int32_t)ceil_div_u((uint64_t)T, QROW_Q);
        // keys per stage of the main scan (qrow_stage_tiles x 64)
        const int64_t stage = kt == ITK_FP8_E4M3 ? 64 : (D * 2 <= 128 ? 512 : (D * 2 <= 256 ? 256 : 128));
        int P = p.G >= 256 ? 1 : (int)ceil_div_u(256, (uint64_t)p.G);
        if (P >= 8) P = (int)ceil_div_u((uint64_t)P, 8) * 8;
        const int Pmax = (int)(N / (4 * stage)) > 1 ? (int)(N / (4 * stage)) : 1;
        if (P > Pmax) P = Pmax;
        if (kn.splits > 0) P = kn.splits;
        if (P > QROW_MAX_SPLITS) P = QROW_MAX_SPLITS;
        int64_t span = (int64_t)ceil_div_u((uint64_t)N, (uint64_t)P);
        span = (int64_t)ceil_div_u((uint64_t)span, (uint64_t)stage) * stage;
        P = (int)ceil_div_u((uint64_t)N, (uint64_t)span);
        p.P = P; p.span = span;
        p.Ps = P; p.span_s = span;
        p.rho = kn.rho > 0.f ? kn.rho : 2.0f;
        // view: about 8 rho k sampled keys per query (between 4096 and 32768)
        double want = 8.0 * p.rho * k;
        if (want < 4096.0) want = 4096.0;
        if (want > 32768.0) want = 32768.0;
        const int64_t ntiles = (int64_t)ceil_div_u((uint64_t)N, TILE_KEYS);
        int64_t st = (int64_t)ceil((double)N / want);
        if (st < 1) st = 1;
        if (st > 4096) st = 4096;
        if (kn.sample_stride > 0) st = kn.sample_stride;
        p.sample_tiles = (int32_t)st;
        p.samp_cap = (int64_t)ceil_div_u((uint64_t)ntiles, (uint64_t)st) * TILE_KEYS;
        // per-(query, split) capacity: 4x the expected share of rho k, >= 64
        int64_t capS = (int64_t)ceil(4.0 * p.rho * k / P);
        if (kn.capacity > 0) capS = (int64_t)ceil_div_u((uint64_t)kn.capacity, (uint64_t)P);
        if (capS < 128) capS = 128;
        capS = (capS + 127) / 128 * 128;  // two halves of a multiple of 64
        p.capS = (int32_t)capS;
        p.cap = (int32_t)(capS * P);
        p.force = kn.force_route;
        size_t off = 0;
        p.off_samp = off; off = align256(off + (size_t)T * p.samp_cap * sizeof(float));
        p.off_gate = off; off = align256(off + (size_t)T * sizeof(float));
        p.off_qcnt = off; off = align256(off + (size_t)T * P * 2 * sizeof(uint32_t));
        p.off_cand = off; off = align256(off + (size_t)T * P * capS * sizeof(Cand));
        p.off_rflag = off; off = align256(off + (size_t)T * sizeof(uint32_t));
        p.bytes = off;
        *out = p;
        return ITK_OK;
    }
    p.G = (int32_t)ceil_div_u((uint64_t)T, FUSED_WAVES);
    // Key splits: fill the 256 CUs with about one workgroup each; a split
    // count that is a multiple of 8 places each split on one XCD.
    int P = p.G >= 256 ? 1 : (int)ceil_div_u(256, (uint64_t)p.G);
    if (P >= 8) P = (int)ceil_div_u((uint64_t)P, 8) * 8;
    const int Pmax = (int)(N / 512) > 1 ? (int)(N / 512) : 1;  // splits of >= 512 keys
    if (P > Pmax) P = Pmax;
    if (kn.splits > 0) P = kn.splits;
    int64_t span = (int64_t)ceil_div_u((uint64_t)N, (uint64_t)P);
    span = (int64_t)ceil_div_u((uint64_t)span, TILE_KEYS) * TILE_KEYS;
    P = (int)ceil_div_u((uint64_t)N, (uint64_t)span);
    p.P = P; p.span = span;
    p.Ps = P; p.span_s = span;
    // Few queries: one key range per wave in the main pass (the sample
    // passes keep the workgroup splits above).  P is a multiple of the waves
    // per workgroup, so that the grid is whole; ranges past N stay empty.
    if (T <= KP_MAX_T && kn.splits == 0) {
        int64_t Pw = (int64_t)ceil_div_u((uint64_t)KP_WAVES, (uint64_t)T);
        int64_t span_w = (int64_t)ceil_div_u((uint64_t)N, (uint64_t)Pw);
        span_w = (int64_t)ceil_div_u((uint64_t)span_w, TILE_KEYS) * TILE_KEYS;
        if (span_w < 4 * TILE_KEYS) span_w = 4 * TILE_KEYS;
        Pw = (int64_t)ceil_div_u((uint64_t)N, (uint64_t)span_w);
        Pw = (int64_t)ceil_div_u((uint64_t)Pw, FUSED_WAVES) * FUSED_WAVES;
        p.kp = true;
        p.P = (int32_t)Pw;
        p.span = span_w;
    }
    const int64_t ntiles = (int64_t)ceil_div_u((uint64_t)N, TILE_KEYS);
    int st = (int)((ntiles + 31) / 32);
    if (st < 1) st = 1;
    if (st > 64) st = 64;
    if (kn.sample_stride > 0) st = kn.sample_stride;
    p.sample_tiles = st;
    p.rho = kn.rho > 0.f ? kn.rho : 2.0f;
    int cap = 4 * k > 2048 ? 4 * k : 2048;
    if (kn.capacity > 0) cap = kn.capacity;
    const int need_all = (int)ceil((double)p.rho * k);
    if (cap < need_all) cap = need_all;
    p.cap = cap;
    p.force = kn.force_route;
    // Pass A stores the view's scores (at most ceil(tiles / stride) tiles per
    // row) when they take no more bytes than the candidate buffer, which
    // keeps the workspace O(T k); a longer view is scored again by pass B.
    p.samp_cap = (int64_t)ceil_div_u((uint64_t)ntiles, (uint64_t)st) * TILE_KEYS;
    if (p.samp_cap > 2 * (int64_t)cap) p.samp_cap = 0;
    if (n_prior > 0) {
        // History sample: the sample passes scan the gathered entries (every
        // one of them, scores stored), split so that about 256 workgroups
        // run, with at least 4 tiles per split.
        p.n_prior = n_prior;
        p.np = (int64_t)ceil_div_u((uint64_t)n_prior, TILE_KEYS) * TILE_KEYS;
        p.rowb = D * (kt == ITK_F32 ? 4 : (kt == ITK_FP8_E4M3 ? 1 : 2));
        int Ps = p.G >= 256 ? 1 : (int)ceil_div_u(256, (uint64_t)p.G);
        const int Psmax = (int)(p.np / (4 * TILE_KEYS)) > 1 ? (int)(p.np / (4 * TILE_KEYS)) : 1;
        if (Ps > Psmax) Ps = Psmax;
        int64_t span_s = (int64_t)ceil_div_u((uint64_t)p.np, (uint64_t)Ps);
        span_s = (int64_t)ceil_div_u((uint64_t)span_s, TILE_KEYS) * TILE_KEYS;
        p.Ps = (int32_t)ceil_div_u((uint64_t)p.np, (uint64_t)span_s);
        p.span_s = span_s;
        p.sample_tiles = 1;
        p.samp_cap = p.np;
    }
    size_t off = 0;
    p.off_param = off; off = align256(off + (size_t)T * sizeof(float4));
    p.off_mm = off; off = align256(off + (size_t)T * p.Ps * sizeof(float2));
    p.off_hist = off; off = align256(off + (size_t)T * NBINS * sizeof(uint32_t));
    p.off_tail = off; off = align256(off + (size_t)T * sizeof(uint32_t));
    p.off_gate = off; off = align256(off + (size_t)T * sizeof(int32_t));
    p.off_cand = off; off = align256(off + (size_t)T * cap * sizeof(Cand));
    p.off_samp = off; off = align256(off + (size_t)T * p.samp_cap * sizeof(float));
    p.off_hist_r = off; off = align256(off + (size_t)T * NBINS * sizeof(uint32_t));
    p.off_rflag = off; off = align256(off + (size_t)T * sizeof(uint32_t));
    p.off_gpub = off; off = align256(off + (size_t)T * sizeof(uint32_t));
    if (n_prior > 0) {
        p.off_pidx = off; off = align256(off + (size_t)p.np * sizeof(int32_t));
        p.off_kp = off; off = align256(off + (size_t)p.np * p.rowb);
        p.off_kps = off; off = align256(off + (size_t)p.np * sizeof(float));
        p.off_pcount = off; off = align256(off + (size_t)T * sizeof(uint32_t));
    }
    p.bytes = off;
    *out = p;
    return ITK_OK;
}

hipError_t launch_fused(const FusedPlan &p, const void *Q, const void *K, const float *k_scale, const float *W,
                        const int32_t *kv_len, int32_t *out_idx, float *out_score, void *ws, hipStream_t stream,
                        const int32_t *prior)
{
    char *w = static_cast<char *>(ws);
    FusedArgs a;
    a.Q = Q; a.K = K; a.k_scale = k_scale; a.W = W; a.kv_len = kv_len;
    a.out_idx = out_idx; a.out_score = out_score;
    const RouteSink &rs = route_sink();
    a.route = (rs.ptr && rs.rows >= p.T) ? rs.ptr : nullptr;
    a.count = (rs.count && rs.count_rows >= p.T) ? rs.count : nullptr;
    a.param = reinterpret_cast<float4 *>(w + p.off_param);
    a.mm = reinterpret_cast<float2 *>(w + p.off_mm);
    a.hist = reinterpret_cast<uint32_t *>(w + p.off_hist);
    a.tail = reinterpret_cast<uint32_t *>(w + p.off_tail);
    a.cand = reinterpret_cast<Cand *>(w + p.off_cand);
    a.N = p.N; a.span = p.span; a.span_s = p.span_s;
    a.T = p.T; a.H = p.H; a.k = p.k; a.cap = p.cap; a.G = p.G; a.P = p.P; a.Ps = p.Ps;
    a.sample_tiles = p.sample_tiles; a.force = p.force; a.rho = p.rho;
    a.samp = p.samp_cap > 0 ? reinterpret_cast<float *>(w + p.off_samp) : nullptr;
    a.hist_r = p.qrow ? nullptr : reinterpret_cast<uint32_t *>(w + p.off_hist_r);
    a.rflag = reinterpret_cast<uint32_t *>(w + p.off_rflag);
    a.gpub = p.qrow ? nullptr : reinterpret_cast<uint32_t *>(w + p.off_gpub);
    a.samp_cap = p.samp_cap;
    a.gate = nullptr; a.qcnt = nullptr; a.capS = 0;
    a.prior = nullptr; a.pidx = nullptr; a.Kp = nullptr; a.kp_scale = nullptr; a.pcount = nullptr;
    a.np = 0; a.n_prior = 0; a.rowb = p.rowb;
    if (p.n_prior > 0) {
        if (!prior || p.qrow) return hipErrorInvalidValue;
        a.prior = prior;
        a.n_prior = p.n_prior;
        a.np = p.np;
        a.pidx = reinterpret_cast<int32_t *>(w + p.off_pidx);
        a.Kp = w + p.off_kp;
        a.kp_scale = k_scale ? reinterpret_cast<float *>(w + p.off_kps) : nullptr;
        a.pcount = reinterpret_cast<uint32_t *>(w + p.off_pcount);
    }
    if (p.qrow) {
        a.gate = reinterpret_cast<float *>(w + p.off_gate);
        a.qcnt = reinterpret_cast<uint32_t *>(w + p.off_qcnt);
        a.cand = reinterpret_cast<Cand *>(w + p.off_cand);
        a.capS = p.capS;
        FusedLauncher fn = find_qrow_launcher(p.qt, p.kt, p.D, !(p.flags & ITK_FLAG_NO_RELU));
        if (!fn) return hipErrorInvalidValue;
        return fn(p, a, stream);
    }
    FusedLauncher fn = find_fused_launcher(p.qt, p.kt, p.HB, p.D, !(p.flags & ITK_FLAG_NO_RELU),
                                           (p.flags & ITK_FLAG_FP8_SCORE) != 0);
    if (!fn) return hipErrorInvalidValue;
    return fn(p, a, stream);
}

// Name of the HIP error behind the last ITK_ERR_HIP of this thread.
static thread_local hipError_t g_last_hip = hipSuccess;

static itk_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return ITK_OK;
    g_last_hip = e;
    return ITK_ERR_HIP;
}

// The padding of rows with no valid key: -1 indices and -inf scores (when
// `score` is given).
__global__ __launch_bounds__(256) void k_fill_pad(int32_t *idx, float *score, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        idx[i] = -1;
        if (score) score[i] = -__builtin_inff();
    }
}

static hipError_t fill_pad(int32_t *idx, float *score, int64_t n, hipStream_t stream)
{
    const int64_t blocks = (n + 255) / 256;
    return launch_kernel(k_fill_pad, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), stream, idx, score,
                         n);
}

bool ragged_trivial(int32_t M, int64_t row_pitch, int32_t k, int32_t *out_idx, hipStream_t stream, itk_status *st)
{
    if (M > 0 && k > 0 && row_pitch > 0) return false;
    if (M < 0 || k < 0 || row_pitch < 0) {
        *st = ITK_ERR_INVALID_ARG;
    } else if (M == 0 || k == 0) {
        *st = ITK_OK;
    } else {
        *st = out_idx ? hip_status(fill_pad(out_idx, nullptr, (int64_t)M * k, stream)) : ITK_ERR_INVALID_ARG;
    }
    return true;
}

// Fused calls with nothing to score.  Returns true when the call is
// complete, with its status in *st.  The shape and dtypes are checked as for
// a non-empty call; then no queries or k == 0 enqueue nothing, and no keys
// (N == 0) leave every row empty, so only the padding is written.
static bool fused_trivial(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k, itk_dtype q_t, itk_dtype k_t,
                          uint32_t flags, int32_t n_prior, int32_t *out_idx, float *out_score, hipStream_t stream,
                          itk_status *st)
{
    if (T > 0 && k > 0 && N > 0) return false;
    if (T < 0 || k < 0 || N < 0) {
        *st = ITK_ERR_INVALID_ARG;
        return true;
    }
    FusedPlan p;
    *st = plan_fused(T > 0 ? T : 1, H, D, N > 0 ? N : 1, k > 0 ? k : 1, q_t, k_t, flags, &p, n_prior);
    if (*st != ITK_OK || T == 0 || k == 0) return true;
    *st = (out_idx && out_score) ? hip_status(fill_pad(out_idx, out_score, (int64_t)T * k, stream))
                                 : ITK_ERR_INVALID_ARG;
    return true;
}

}  // namespace itk

using namespace itk;

extern "C" {


const char *itk_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

const char *itk_status_string(itk_status s)
{
    switch (s) {
    case ITK_OK: return "ok";
    case ITK_ERR_INVALID_ARG: return "invalid argument";
    case ITK_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case ITK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ITK_ERR_HIP: return "HIP runtime error";
    case ITK_ERR_SCRATCH_LIMIT: return "shape needs more than the static scratch of the no-allocation call";
    default: return "unknown status";
    }
}

size_t topk_ragged_workspace_size(int32_t M, int64_t row_pitch, int32_t k)
{
    if (M <= 0 || row_pitch <= 0 || k <= 0 || row_pitch > (int64_t)0x7FFFFFFF) return 0;
    return plan_ragged(M, row_pitch, k).bytes;
}

itk_status topk_ragged(const float *scores, int64_t row_pitch, const int32_t *row_len, int32_t M, int32_t k,
                       int32_t *out_idx, void *workspace, size_t workspace_bytes, void *stream)
{
    itk_status st;
    if (ragged_trivial(M, row_pitch, k, out_idx, static_cast<hipStream_t>(stream), &st)) return st;
    if (!scores || !row_len || !out_idx) return ITK_ERR_INVALID_ARG;
    if (row_pitch > (int64_t)0x7FFFFFFF) return ITK_ERR_UNSUPPORTED;
    const RaggedPlan p = plan_ragged(M, row_pitch, k);
    if (!workspace || workspace_bytes < p.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return ITK_ERR_WORKSPACE;
    const hipError_t e = launch_ragged(p, scores, row_len, out_idx, workspace, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

size_t indexer_topk_fused_workspace_size(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k, itk_dtype q_t,
                                         itk_dtype k_t, uint32_t flags)
{
    FusedPlan p;
    if (plan_fused(T, H, D, N, k, q_t, k_t, flags, &p) != ITK_OK) return 0;
    return p.bytes;
}

itk_status indexer_topk_fused(const void *Q, itk_dtype q_t, const void *K, itk_dtype k_t, const float *k_scale,
                              const float *W, const int32_t *kv_len, int32_t T, int32_t H, int32_t D, int64_t N,
                              int32_t k, uint32_t flags, int32_t *out_idx, float *out_score, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    itk_status st;
    if (fused_trivial(T, H, D, N, k, q_t, k_t, flags, 0, out_idx, out_score, static_cast<hipStream_t>(stream), &st))
        return st;
    if (!Q || !K || !W || !kv_len || !out_idx || !out_score) return ITK_ERR_INVALID_ARG;
    if ((k_t == ITK_FP8_E4M3) != (k_scale != nullptr)) return ITK_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(Q) & 15u) || (reinterpret_cast<uintptr_t>(K) & 15u)) return ITK_ERR_INVALID_ARG;
    FusedPlan p;
    st = plan_fused(T, H, D, N, k, q_t, k_t, flags, &p);
    if (st != ITK_OK) return st;
    if (!workspace || workspace_bytes < p.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return ITK_ERR_WORKSPACE;
    const hipError_t e = launch_fused(p, Q, K, k_scale, W, kv_len, out_idx, out_score, workspace,
                                      static_cast<hipStream_t>(stream));
    return hip_status(e);
}

size_t indexer_topk_fused_prior_workspace_size(int32_t T, int32_t H, int32_t D, int64_t N, int32_t k,
                                               itk_dtype q_t, itk_dtype k_t, uint32_t flags, int32_t n_prior)
{
    FusedPlan p;
    if (plan_fused(T, H, D, N, k, q_t, k_t, flags, &p, n_prior) != ITK_OK) return 0;
    return p.bytes;
}

itk_status indexer_topk_fused_prior(const void *Q, itk_dtype q_t, const void *K, itk_dtype k_t,
                                    const float *k_scale, const float *W, const int32_t *kv_len, int32_t T,
                                    int32_t H, int32_t D, int64_t N, int32_t k, uint32_t flags,
                                    const int32_t *prior_idx, int32_t n_prior, int32_t *out_idx, float *out_score,
                                    void *workspace, size_t workspace_bytes, void *stream)
{
    itk_status st;
    if (n_prior < 0) return ITK_ERR_INVALID_ARG;
    if (fused_trivial(T, H, D, N, k, q_t, k_t, flags, n_prior, out_idx, out_score, static_cast<hipStream_t>(stream),
                      &st))
        return st;
    if (!Q || !K || !W || !kv_len || !out_idx || !out_score) return ITK_ERR_INVALID_ARG;
    if ((k_t == ITK_FP8_E4M3) != (k_scale != nullptr)) return ITK_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(Q) & 15u) || (reinterpret_cast<uintptr_t>(K) & 15u)) return ITK_ERR_INVALID_ARG;
    if (n_prior > 0 && !prior_idx) return ITK_ERR_INVALID_ARG;
    FusedPlan p;
    st = plan_fused(T, H, D, N, k, q_t, k_t, flags, &p, n_prior);
    if (st != ITK_OK) return st;
    if (!workspace || workspace_bytes < p.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return ITK_ERR_WORKSPACE;
    const hipError_t e = launch_fused(p, Q, K, k_scale, W, kv_len, out_idx, out_score, workspace,
                                      static_cast<hipStream_t>(stream), prior_idx);
    return hip_status(e);
}

size_t indexer_prior_workspace_size(int32_t T_prev, int32_t k, int64_t N, int32_t k_prime)
{
    PriorPlan p;
    if (plan_prior(T_prev, k, N, k_prime, &p) != ITK_OK) return 0;
    return p.bytes;
}

itk_status indexer_prior_from_topk(const int32_t *prev_idx, int32_t T_prev, int32_t k, int64_t N, int32_t k_prime,
                                   int32_t *prior_out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!prior_out || (T_prev > 0 && !prev_idx)) return ITK_ERR_INVALID_ARG;
    PriorPlan p;
    const itk_status st = plan_prior(T_prev, k, N, k_prime, &p);
    if (st != ITK_OK) return st;
    if (!workspace || workspace_bytes < p.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return ITK_ERR_WORKSPACE;
    return hip_status(launch_prior(p, prev_idx, prior_out, workspace, static_cast<hipStream_t>(stream)));
}

itk_status itk_set_plan_opts(const itk_plan_opts *o)
{
    Knobs &k = knobs();
    if (!o) {
        k = Knobs();
        return ITK_OK;
    }
    if (o->sample_stride < 0 || o->capacity < 0 || o->splits < 0 || o->force_route < 0 || o->force_route > 2 ||
        o->ragged_route < 0 || o->ragged_route > 3 ||
        !(o->rho >= 0.f) || !(o->rho1 >= 0.f))
        return ITK_ERR_INVALID_ARG;
    if (o->sample_stride > 0 && o->sample_stride > 4096) return ITK_ERR_INVALID_ARG;
    k.sample_stride = o->sample_stride;
    k.rho = o->rho;
    k.rho1 = o->rho1;
    k.capacity = o->capacity;
    k.splits = o->splits;
    k.force_route = o->force_route;
    k.route_select = o->ragged_route;
    return ITK_OK;
}

itk_status itk_set_route_buffer(int32_t *route_out, int32_t rows)
{
    if (route_out && rows <= 0) return ITK_ERR_INVALID_ARG;
    route_sink().ptr = route_out;
    route_sink().rows = route_out ? rows : 0;
    return ITK_OK;
}

itk_status itk_set_count_buffer(int32_t *count_out, int32_t rows)
{
    if (count_out && rows <= 0) return ITK_ERR_INVALID_ARG;
    route_sink().count = count_out;
    route_sink().count_rows = count_out ? rows : 0;
    return ITK_OK;
}

itk_status itk_profile_enable(int32_t on)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
    return ITK_OK;
}

int32_t itk_profile_read(double *ms_out, int32_t *count_out, const char **names_out, int32_t max_stages)
{
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof);
    }
    double ms[ST_COUNT] = {0};
    int32_t cnt[ST_COUNT] = {0};
    for (const ProfRec &r : recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
            ms[r.stage] += t;
            cnt[r.stage] += 1;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    const int n = max_stages < ST_COUNT ? max_stages : ST_COUNT;
    for (int i = 0; i < n; ++i) {
        if (ms_out) ms_out[i] = ms[i];
        if (count_out) count_out[i] = cnt[i];
        if (names_out) names_out[i] = g_stage_names[i];
    }
    return n;
}

}  // extern "C"
