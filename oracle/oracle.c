/*
 * CPU oracle for the fused Indexer-TopK and the standalone ragged Top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or constant with the HIP library: the formats are decoded here from their
 * published definitions, the score is the plain sum, and selection is a full
 * sort.  Nothing here is blocked, fused or reordered.
 *
 * What it computes (the plain definitions):
 *
 *  - Lightning-indexer score (LiteTopK, Sec. 2.1, Eq. (1)):
 *        I[t,j] = sum_h w[t,h] * ReLU( q[t,h,:] . k[j,:] )
 *    over the causally valid keys j < kv_len[t].  Weights are per query
 *    (Eq. (1) indexes them by t).  With the NO_RELU flag and H = 1 the score
 *    is the plain inner product q[t,0,:] . k[j,:] (the k-NN case of the
 *    problem definition, LiteTopK Sec. 3.1 Eq. (2)).
 *    FP8 keys are dequantised as decode(k8[j,d]) * scale[j].
 *    Arithmetic: every input is widened exactly to double; products and sums
 *    are accumulated in double, sequentially over d and then over h.
 *    Valid lengths are clamped: L_t = min(max(kv_len[t], 0), N).
 *
 *  - FP8 scoring (the FP8_SCORE flag, FP8 keys only): the DSA indexer of
 *    LiteTopK Sec. 2.1 multiplies FP8 queries with FP8 keys.  Each
 *    (query, head) row q[t,h,:] is quantized on its own: with
 *    a = max_d |q[t,h,d]| > 0, the code of element d is the e4m3fn value
 *    nearest (ties to even) to q[t,h,d] * (448 / a), where 448 / a and the
 *    product are each rounded to fp32 (the code is an integer decision, so
 *    it is taken in the precision the kernel takes it in), and the row's
 *    scale is s = a / 448 rounded to fp32 (a row of zeros keeps code 0 and
 *    s = 1).  The score is then Eq. (1) over the dequantized rows,
 *        I[t,j] = sum_h w[t,h] * s[t,h] * ReLU( code[t,h,:] . k[j,:] ),
 *    summed in double like the plain score.
 *
 *  - Exact Top-k (LiteTopK Sec. 3.1 Eq. (2); the exactness criterion of the
 *    Sample-Guided Exact Top-K paper, Sec. 6.1 Eq. (30)): sort the valid
 *    entries of a row by (score descending, index ascending) and keep the
 *    first min(k, L).  Equal scores (including -0 == +0) go to the lower
 *    index.  Output slots past min(k, L) hold index -1.
 *
 *  - History sample (LiteTopK Sec. 3.2 "Sampling"): the k' keys that occur
 *    most often in the previous chunk's Top-k lists.  Count, for every key
 *    j in [0, N), the entries of the previous lists equal to j (entries
 *    outside [0, N), such as -1 padding, count for nothing); sort the keys by
 *    (count descending, index ascending) and keep the first min(k', N).
 *    Output slots past that hold -1.  The prior only places the initial gate
 *    of the fused call; it never changes the fused Top-k.
 *
 * Formats (decoded from their definitions, not by bit reinterpretation):
 *  - bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 *  - fp16 (IEEE-754 binary16): 1 sign, 5 exponent (bias 15), 10 fraction bits.
 *  - e4m3fn (OCP 8-bit floating point, E4M3): 1 sign, 4 exponent (bias 7),
 *    3 fraction bits, no infinities, S.1111.111 is NaN, largest finite 448.
 *    Encoding rounds to the nearest value, ties to the even fraction; a
 *    magnitude that rounds above 448 (i.e. above 464), inf and NaN give NaN.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_F16 = 2, ORA_FP8_E4M3 = 3 };
enum { ORA_FLAG_NO_RELU = 1, ORA_FLAG_FP8_SCORE = 2 };

/* Generic binary floating-point decode: sign bit, ebits exponent bits,
 * mbits fraction bits, bias; `has_inf` selects IEEE-style inf/NaN at the top
 * exponent, otherwise only the all-ones code is NaN (e4m3fn). */
static double decode_generic(uint32_t bits, int ebits, int mbits, int bias, int has_inf)
{
    uint32_t sign = (bits >> (ebits + mbits)) & 1u;
    uint32_t e = (bits >> mbits) & ((1u << ebits) - 1u);
    uint32_t m = bits & ((1u << mbits) - 1u);
    uint32_t emax = (1u << ebits) - 1u;
    double v;
    if (has_inf && e == emax) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (!has_inf && e == emax && m == (1u << mbits) - 1u) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)m / (double)(1u << mbits), 1 - bias);
    } else {
        v = ldexp(1.0 + (double)m / (double)(1u << mbits), (int)e - bias);
    }
    return sign ? -v : v;
}

double ora_decode(int dtype, uint32_t bits)
{
    switch (dtype) {
    case ORA_BF16: return decode_generic(bits & 0xFFFFu, 8, 7, 127, 1);
    case ORA_F16: return decode_generic(bits & 0xFFFFu, 5, 10, 15, 1);
    case ORA_FP8_E4M3: return decode_generic(bits & 0xFFu, 4, 3, 7, 0);
    case ORA_F32: {
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    default: return NAN;
    }
}

void ora_decode_array(int dtype, const void *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = 0;
        if (dtype == ORA_F32) b = ((const uint32_t *)src)[i];
        else if (dtype == ORA_FP8_E4M3) b = ((const uint8_t *)src)[i];
        else b = ((const uint16_t *)src)[i];
        dst[i] = ora_decode(dtype, b);
    }
}

/* e4m3fn encoding of an fp32 value, from the format's value set: the
 * magnitude is divided by the spacing of its binade (2^-9 below the smallest
 * normal 2^-6, else 2^(e-3) for 2^e <= |x| < 2^(e+1)), which is exact in
 * double, rounded to the nearest integer with ties to even (rint under the
 * default rounding mode), and scaled back; the result is then written as
 * sign, biased exponent and fraction.  Results above 448 are NaN (0x7F). */
uint8_t ora_encode_e4m3(float x)
{
    const double v = (double)x;
    const uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
    const double a = fabs(v);
    if (isinf(a)) return (uint8_t)(sign | 0x7Fu);
    const double min_normal = ldexp(1.0, -6);
    double spacing;
    if (a < min_normal) {
        spacing = ldexp(1.0, -9);
    } else {
        int e;
        (void)frexp(a, &e);          /* a = f * 2^e, 0.5 <= f < 1 */
        spacing = ldexp(1.0, (e - 1) - 3);
    }
    const double r = rint(a / spacing) * spacing;
    if (r > 448.0) return (uint8_t)(sign | 0x7Fu);
    if (r == 0.0) return sign;
    if (r < min_normal) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));  /* subnormal */
    int e;
    const double f = frexp(r, &e);   /* r = (2 f) * 2^(e-1), 1 <= 2f < 2 */
    const int E = (e - 1) + 7;
    const int m = (int)((2.0 * f - 1.0) * 8.0);
    return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)m);
}

typedef struct { const float *src; uint8_t *dst; int64_t n, lo, hi; } enc_job_t;

static void *enc_worker(void *p)
{
    enc_job_t *j = (enc_job_t *)p;
    for (int64_t i = j->lo; i < j->hi; ++i) j->dst[i] = ora_encode_e4m3(j->src[i]);
    return NULL;
}

/* Encodes n values, split over `nthreads` threads. */
void ora_encode_e4m3_array(const float *src, uint8_t *dst, int64_t n, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    pthread_t th[64];
    enc_job_t jobs[64];
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (enc_job_t){src, dst, n, n * i / nthreads, n * (i + 1) / nthreads};
        if (pthread_create(&th[started], NULL, enc_worker, &jobs[i]) == 0) ++started;
        else enc_worker(&jobs[i]);
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
}

/* ---- decode tables (built once from ora_decode) --------------------------- */
static double g_lut16[3][65536];
static double g_lut8[256];
static pthread_once_t g_lut_once = PTHREAD_ONCE_INIT;
static void build_luts(void)
{
    for (uint32_t b = 0; b < 65536u; ++b) {
        g_lut16[ORA_BF16][b] = ora_decode(ORA_BF16, b);
        g_lut16[ORA_F16][b] = ora_decode(ORA_F16, b);
    }
    for (uint32_t b = 0; b < 256u; ++b) g_lut8[b] = ora_decode(ORA_FP8_E4M3, b);
}

static inline double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORA_F32) return (double)((const float *)base)[i];
    if (dtype == ORA_FP8_E4M3) return g_lut8[((const uint8_t *)base)[i]];
    return g_lut16[dtype][((const uint16_t *)base)[i]];
}

typedef struct {
    const void *Q; int q_t;
    const void *K; int k_t;
    const float *k_scale;
    const float *W;
    int H, D;
    int64_t N;
    uint32_t flags;
} fused_args;

/* L_t = min(max(kv_len[t], 0), N). */
static int64_t valid_len(int64_t kv, int64_t N)
{
    if (kv < 0) return 0;
    return kv > N ? N : kv;
}

/* Query rows widened once: qbuf[h*D + d] = q[t,h,d] and hfac[h] = 1; with
 * FP8 scoring, qbuf holds the decoded e4m3fn codes of each (t,h) row and
 * hfac[h] its fp32 scale a / 448 (see the header for the quantization). */
static void load_query(const fused_args *a, int t, double *qbuf, double *hfac)
{
    for (int h = 0; h < a->H; ++h) {
        for (int d = 0; d < a->D; ++d)
            qbuf[h * a->D + d] = elem(a->Q, a->q_t, ((int64_t)t * a->H + h) * a->D + d);
        hfac[h] = 1.0;
        if (!(a->flags & ORA_FLAG_FP8_SCORE)) continue;
        float amax = 0.0f;  /* the inputs are bf16/fp16/fp32 values: exact in float */
        for (int d = 0; d < a->D; ++d) {
            const float x = (float)fabs(qbuf[h * a->D + d]);
            if (x > amax) amax = x;
        }
        const int usable = amax > 0.0f && isfinite(amax);
        const float inv = usable ? 448.0f / amax : 0.0f;
        for (int d = 0; d < a->D; ++d) {
            const float y = (float)qbuf[h * a->D + d] * inv;  /* fp32 product */
            qbuf[h * a->D + d] = ora_decode(ORA_FP8_E4M3, ora_encode_e4m3(y));
        }
        hfac[h] = usable ? (double)(amax / 448.0f) : 1.0;
    }
}

/* I[t,j]: the definition, in double (sequential over d, then over h). */
static double score_key(const fused_args *a, const double *qbuf, const double *hfac, int t, int64_t j,
                        double *kbuf)
{
    const int H = a->H, D = a->D;
    const double sc = (a->k_t == ORA_FP8_E4M3 && a->k_scale) ? (double)a->k_scale[j] : 1.0;
    for (int d = 0; d < D; ++d) kbuf[d] = elem(a->K, a->k_t, j * D + d) * sc;
    double s = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qbuf[h * D + d] * kbuf[d];
        const double w = (double)a->W[(int64_t)t * H + h] * hfac[h];
        if (a->flags & ORA_FLAG_NO_RELU) s += w * dot;
        else s += w * (dot > 0.0 ? dot : 0.0);
    }
    return s;
}

/* Full score row of query t over keys [0, L). */
static void score_row(const fused_args *a, int t, int64_t L, double *out, double *qbuf, double *hfac,
                      double *kbuf)
{
    load_query(a, t, qbuf, hfac);
    for (int64_t j = 0; j < L; ++j) out[j] = score_key(a, qbuf, hfac, t, j, kbuf);
}

/* ---- selection: full sort by (value desc, index asc) ----------------------- */
typedef struct { double v; int64_t i; } vi_t;

static int cmp_vi(const void *pa, const void *pb)
{
    const vi_t *a = (const vi_t *)pa, *b = (const vi_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* Returns min(k, L); writes indices of the top min(k, L) in sorted order,
 * pads the rest of out_idx[0..k) with -1, and (optionally) their scores. */
static int select_sorted(vi_t *buf, int64_t L, int k, int32_t *out_idx, double *out_val)
{
    qsort(buf, (size_t)L, sizeof(vi_t), cmp_vi);
    int n = (L < k) ? (int)L : k;
    for (int r = 0; r < k; ++r) {
        if (r < n) {
            out_idx[r] = (int32_t)buf[r].i;
            if (out_val) out_val[r] = buf[r].v;
        } else {
            out_idx[r] = -1;
            if (out_val) out_val[r] = -INFINITY;
        }
    }
    return n;
}

int ora_select_f64(const double *s, int64_t L, int k, int32_t *out_idx, double *out_val)
{
    if (L < 0 || k <= 0) return -1;
    vi_t *buf = (vi_t *)malloc(sizeof(vi_t) * (size_t)(L > 0 ? L : 1));
    if (!buf) return -2;
    for (int64_t j = 0; j < L; ++j) { buf[j].v = s[j]; buf[j].i = j; }
    int n = select_sorted(buf, L, k, out_idx, out_val);
    free(buf);
    return n;
}

int ora_select_f32(const float *s, int64_t L, int k, int32_t *out_idx)
{
    if (L < 0 || k <= 0) return -1;
    vi_t *buf = (vi_t *)malloc(sizeof(vi_t) * (size_t)(L > 0 ? L : 1));
    if (!buf) return -2;
    for (int64_t j = 0; j < L; ++j) { buf[j].v = (double)s[j]; buf[j].i = j; }
    int n = select_sorted(buf, L, k, out_idx, NULL);
    free(buf);
    return n;
}

/* ---- threaded drivers: one worker per core, rows handed out in order ------ */
typedef struct {
    /* fused */
    fused_args fa;
    const int32_t *kv_len;
    /* ragged */
    const float *scores;
    int64_t pitch;
    const int32_t *row_len;
    /* common */
    const int32_t *rows;
    int nrows, k;
    int32_t *out_idx;
    double *out_val;
    int32_t *out_n;
    int64_t maxL;
    int next;
    int status;
    pthread_mutex_t mu;
} job_t;

static int take_row(job_t *j)
{
    pthread_mutex_lock(&j->mu);
    int r = j->next < j->nrows ? j->next++ : -1;
    pthread_mutex_unlock(&j->mu);
    return r;
}

static void *fused_worker(void *p)
{
    job_t *j = (job_t *)p;
    const int H = j->fa.H, D = j->fa.D;
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *hfac = (double *)malloc(sizeof(double) * (size_t)H);
    double *kbuf = (double *)malloc(sizeof(double) * (size_t)D);
    double *row = (double *)malloc(sizeof(double) * (size_t)(j->maxL > 0 ? j->maxL : 1));
    vi_t *buf = (vi_t *)malloc(sizeof(vi_t) * (size_t)(j->maxL > 0 ? j->maxL : 1));
    if (!qbuf || !hfac || !kbuf || !row || !buf) { j->status = -2; goto out; }
    for (int r; (r = take_row(j)) >= 0;) {
        int t = j->rows[r];
        int64_t L = valid_len(j->kv_len[t], j->fa.N);
        score_row(&j->fa, t, L, row, qbuf, hfac, kbuf);
        for (int64_t x = 0; x < L; ++x) { buf[x].v = row[x]; buf[x].i = x; }
        j->out_n[r] = select_sorted(buf, L, j->k, j->out_idx + (int64_t)r * j->k,
                                    j->out_val ? j->out_val + (int64_t)r * j->k : NULL);
    }
out:
    free(qbuf); free(hfac); free(kbuf); free(row); free(buf);
    return NULL;
}

static void *ragged_worker(void *p)
{
    job_t *j = (job_t *)p;
    vi_t *buf = (vi_t *)malloc(sizeof(vi_t) * (size_t)(j->maxL > 0 ? j->maxL : 1));
    if (!buf) { j->status = -2; return NULL; }
    for (int r; (r = take_row(j)) >= 0;) {
        int m = j->rows[r];
        const int64_t L = valid_len(j->row_len[m], j->pitch);
        const float *x = j->scores + (int64_t)m * j->pitch;
        for (int64_t i = 0; i < L; ++i) { buf[i].v = (double)x[i]; buf[i].i = i; }
        j->out_n[r] = select_sorted(buf, L, j->k, j->out_idx + (int64_t)r * j->k, NULL);
    }
    free(buf);
    return NULL;
}

static int run_threads(job_t *j, void *(*fn)(void *), int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    pthread_mutex_init(&j->mu, NULL);
    j->next = 0;
    j->status = 0;
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, j) == 0) ++started;
    if (started == 0) fn(j);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&j->mu);
    return j->status;
}

/* Top-k of the fused score for the listed query rows of a call with N keys.
 * out_idx/out_val: [nrows, k]; out_n: [nrows] = min(k, L_t). */
int ora_fused_topk(const void *Q, int q_t, const void *K, int k_t, const float *k_scale,
                   const float *W, const int32_t *kv_len, int64_t N, int H, int D, uint32_t flags,
                   const int32_t *rows, int nrows, int k, int32_t *out_idx, double *out_val,
                   int32_t *out_n, int nthreads)
{
    pthread_once(&g_lut_once, build_luts);
    if (k <= 0 || H <= 0 || D <= 0 || N < 0 || nrows < 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.fa = (fused_args){Q, q_t, K, k_t, k_scale, W, H, D, N, flags};
    j.kv_len = kv_len;
    j.rows = rows; j.nrows = nrows; j.k = k;
    j.out_idx = out_idx; j.out_val = out_val; j.out_n = out_n;
    for (int r = 0; r < nrows; ++r) {
        const int64_t L = valid_len(kv_len[rows[r]], N);
        if (L > j.maxL) j.maxL = L;
    }
    return run_threads(&j, fused_worker, nthreads);
}

/* Score of single (query, key) pairs: out[i] = I[t[i], j[i]], for keys
 * 0 <= j[i] < N (any other key index is rejected with -1). */
int ora_fused_scores_at(const void *Q, int q_t, const void *K, int k_t, const float *k_scale,
                        const float *W, int64_t N, int H, int D, uint32_t flags, const int32_t *t_idx,
                        const int64_t *j_idx, int64_t n, double *out)
{
    pthread_once(&g_lut_once, build_luts);
    for (int64_t i = 0; i < n; ++i)
        if (j_idx[i] < 0 || j_idx[i] >= N) return -1;
    fused_args a = {Q, q_t, K, k_t, k_scale, W, H, D, N, flags};
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *hfac = (double *)malloc(sizeof(double) * (size_t)H);
    double *kbuf = (double *)malloc(sizeof(double) * (size_t)D);
    if (!qbuf || !hfac || !kbuf) { free(qbuf); free(hfac); free(kbuf); return -2; }
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || t_idx[i] != t_idx[i - 1]) load_query(&a, t_idx[i], qbuf, hfac);
        out[i] = score_key(&a, qbuf, hfac, t_idx[i], j_idx[i], kbuf);
    }
    free(qbuf); free(hfac); free(kbuf);
    return 0;
}

/* Full score row of query t over keys [0, min(max(L, 0), N)); returns the
 * number of scores written. */
int64_t ora_fused_score_row(const void *Q, int q_t, const void *K, int k_t, const float *k_scale,
                            const float *W, int64_t N, int H, int D, uint32_t flags, int t, int64_t L,
                            double *out)
{
    pthread_once(&g_lut_once, build_luts);
    fused_args a = {Q, q_t, K, k_t, k_scale, W, H, D, N, flags};
    L = valid_len(L, N);
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *hfac = (double *)malloc(sizeof(double) * (size_t)H);
    double *kbuf = (double *)malloc(sizeof(double) * (size_t)D);
    if (!qbuf || !hfac || !kbuf) { free(qbuf); free(hfac); free(kbuf); return -2; }
    score_row(&a, t, L, out, qbuf, hfac, kbuf);
    free(qbuf); free(hfac); free(kbuf);
    return L;
}

/* Standalone exact Top-k of the listed rows of a [M, pitch] fp32 matrix. */
int ora_topk_ragged(const float *scores, int64_t pitch, const int32_t *row_len,
                    const int32_t *rows, int nrows, int k, int32_t *out_idx, int32_t *out_n,
                    int nthreads)
{
    if (k <= 0 || pitch < 0 || nrows < 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.scores = scores; j.pitch = pitch; j.row_len = row_len;
    j.rows = rows; j.nrows = nrows; j.k = k;
    j.out_idx = out_idx; j.out_n = out_n;
    j.maxL = pitch;
    return run_threads(&j, ragged_worker, nthreads);
}

/* History sample: the k_prime most frequent keys of the previous chunk's
 * Top-k lists prev_idx[T_prev][k] (count descending, index ascending). */
int ora_prior_from_topk(const int32_t *prev_idx, int64_t T_prev, int k, int64_t N, int k_prime,
                        int32_t *out)
{
    if (T_prev < 0 || k <= 0 || N <= 0 || k_prime <= 0) return -1;
    vi_t *buf = (vi_t *)malloc(sizeof(vi_t) * (size_t)N);
    if (!buf) return -2;
    for (int64_t j = 0; j < N; ++j) { buf[j].v = 0.0; buf[j].i = j; }
    for (int64_t e = 0; e < T_prev * (int64_t)k; ++e) {
        const int64_t j = prev_idx[e];
        if (j >= 0 && j < N) buf[j].v += 1.0;
    }
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)k_prime);
    if (!tmp) { free(buf); return -2; }
    const int n = select_sorted(buf, N, k_prime, tmp, NULL);
    memcpy(out, tmp, sizeof(int32_t) * (size_t)k_prime);
    free(tmp);
    free(buf);
    return n;
}
