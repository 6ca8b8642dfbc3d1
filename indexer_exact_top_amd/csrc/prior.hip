// History sample for the fused Indexer-TopK (LiteTopK, Sec. 3.2 "Sampling"):
// the k' keys that occur most often in the previous chunk's Top-k lists.
//
// Prefix keys are shared across the chunks of a prefill, and adjacent chunks
// tend to attend to the same prefix tokens, so these keys are likely to score
// high again; scored first, they give the next chunk a tight initial gate.
//
// The selection is by (count descending, index ascending) over the integer
// counts, so it needs no floating point and no general Top-k:
//  1. count: workgroup (r, s) counts the entries of list slice s that fall in
//     key range r into LDS counters, then adds its non-zero counters to the
//     global counts (one global atomic per key and slice, not per entry: a
//     key popular with every query appears once per list).  Every slice is
//     read once per key range, so past P_MAX_RANGES ranges each entry adds
//     to its key's global count directly instead;
//  2. threshold: a two-level histogram (count >> 12, then count & 4095 within
//     the boundary bin) gives the k''-th largest count c* exactly
//     (k'' = min(k', N)), the number of keys above it, and the quota of keys
//     equal to c* that are taken (the lowest indices);
//  3. emit: per block of keys, the numbers above and equal to c*, one prefix
//     over the blocks, then every taken key is written at its rank in index
//     order, so the list comes out in ascending index order.
#include "itk_internal.hpp"
#include "itk_device.hpp"

namespace itk {

namespace {

constexpr int PT = 1024;              // threads per workgroup
constexpr int P_RANGE = 32768;        // keys per counting range (LDS counters)
constexpr int64_t P_SLICE = 65536;    // list entries per counting workgroup
constexpr int P_HB1 = 8192;           // level-1 bins: count >> 12 (counts < 2^25)
constexpr int P_HB2 = 4096;           // level-2 bins: count & 4095
constexpr int P_BLK = 4 * PT;         // keys per emission block (4 per thread)
constexpr int64_t P_MAX_ENTRIES = ((int64_t)1 << 25) - 1;
// Key ranges up to which the LDS counting pays for re-reading the lists
// (measured: 0.074 against 0.168 ms at 5 ranges, 0.230 against 0.204 ms at
// 32, 0.72 against 0.23 ms at 128).
constexpr int P_MAX_RANGES = 16;

struct PriorArgs {
    const int32_t *prev;  // [n_entries] previous lists
    int64_t n_entries;
    uint32_t *cnt;        // [N] occurrence counts
    uint32_t *h1;         // [P_HB1]
    uint32_t *h2;         // [P_HB2]
    uint32_t *blk;        // [nblk][2] per block (above c*, equal to c*), then their exclusive prefixes
    uint32_t *par;        // [0] b1, [1] keys above bin b1, [2] c*, [3] keys above c*, [4] quota at c*
    int32_t *out;         // [k_prime]
    int64_t N;
    int32_t k_prime, kk, nblk, nrange;
};

// Workgroup-wide exclusive prefix of one value per thread (PT threads).
// `ws` holds PT / 64 words.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t *ws, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t incl = wave_incl_sum(v);
    __syncthreads();
    if (lane == 63) ws[wave] = incl;
    __syncthreads();
    uint32_t off = 0, all = 0;
    for (int w = 0; w < PT / 64; ++w) {
        const uint32_t x = ws[w];
        off += w < wave ? x : 0u;
        all += x;
    }
    *total = all;
    return off + incl - v;
}

// The largest bin b with (base + sum_{b' >= b} hist[b']) >= need, and the
// count strictly above it (base included), over NB bins read from global
// memory; every thread returns the same values.  Requires base < need <=
// base + sum(hist).
template <int NB>
__device__ __forceinline__ void top_bin(const uint32_t *hist, uint32_t base, uint32_t need, uint32_t *ws,
                                        uint32_t *s_out, int *b_out, uint32_t *above_out)
{
    constexpr int PER = NB / PT;
    const int tid = threadIdx.x;
    uint32_t h[PER], mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        h[i] = hist[tid * PER + i];
        mine += h[i];
    }
    // suffix over threads: sum of the bins of every higher thread
    uint32_t total;
    const uint32_t before = block_excl_sum(mine, ws, &total);
    uint32_t run = base + (total - before - mine);
    if (tid == 0) s_out[0] = 0xFFFFFFFFu;
    __syncthreads();
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
        const uint32_t prev = run;
        run += h[i];
        if (prev < need && run >= need) {  // exactly one bin crosses
            s_out[0] = (uint32_t)(tid * PER + i);
            s_out[1] = prev;
        }
    }
    __syncthreads();
    *b_out = (int)s_out[0];
    *above_out = s_out[1];
}

__global__ __launch_bounds__(PT) void k_prior_clear(PriorArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * PT;
    for (int64_t i = (int64_t)blockIdx.x * PT + threadIdx.x; i < a.N; i += stride) a.cnt[i] = 0u;
    const int64_t g = (int64_t)blockIdx.x * PT + threadIdx.x;
    if (g < P_HB1) a.h1[g] = 0u;
    if (g < P_HB2) a.h2[g] = 0u;
}

// Workgroup (range r, slice s) = blockIdx.x = r + nrange * s.
__global__ __launch_bounds__(PT) void k_prior_count(PriorArgs a)
{
    __shared__ uint32_t c[P_RANGE];
    const int tid = threadIdx.x;
    const int r = (int)(blockIdx.x % (unsigned)a.nrange), s = (int)(blockIdx.x / (unsigned)a.nrange);
    for (int i = tid; i < P_RANGE; i += PT) c[i] = 0u;
    __syncthreads();
    const int64_t lo = (int64_t)r * P_RANGE;
    const int64_t hi = lo + P_RANGE < a.N ? lo + P_RANGE : a.N;
    const int64_t e0 = (int64_t)s * P_SLICE;
    const int64_t e1 = e0 + P_SLICE < a.n_entries ? e0 + P_SLICE : a.n_entries;
    constexpr int U = 8;  // loads in flight per thread
    for (int64_t e = e0 + tid; e < e1; e += (int64_t)PT * U) {
        int64_t j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = e + (int64_t)u * PT < e1 ? (int64_t)a.prev[e + (int64_t)u * PT] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j[u] >= lo && j[u] < hi) atomicAdd(&c[j[u] - lo], 1u);
    }
    __syncthreads();
    for (int i = tid; lo + i < hi; i += PT) {
        const uint32_t v = c[i];
        if (v) atomicAdd(&a.cnt[lo + i], v);
    }
}

// Counting for many key ranges: one global atomic per list entry.
__global__ __launch_bounds__(PT) void k_prior_count_direct(PriorArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * PT;
    for (int64_t e = (int64_t)blockIdx.x * PT + threadIdx.x; e < a.n_entries; e += stride) {
        const int64_t j = a.prev[e];
        if (j >= 0 && j < a.N) atomicAdd(&a.cnt[j], 1u);
    }
}

// Adds 1 to bin b of an LDS histogram; the lanes of a wave that hit bin 0
// (the counts of most keys) add with one atomic.
__device__ __forceinline__ void hist_add(uint32_t *h, uint32_t b, bool valid)
{
    const uint64_t zero = __ballot(valid && b == 0u);
    if (zero && lane_id() == (uint32_t)__builtin_ctzll(zero)) atomicAdd(&h[0], (uint32_t)__popcll(zero));
    if (valid && b != 0u) atomicAdd(&h[b], 1u);
}

// Level 1: histogram of count >> 12 over a block of keys.
__global__ __launch_bounds__(PT) void k_prior_hist1(PriorArgs a)
{
    __shared__ uint32_t h[P_HB1];
    const int tid = threadIdx.x;
    for (int i = tid; i < P_HB1; i += PT) h[i] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * P_BLK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = base + (int64_t)i * PT + tid;
        const bool ok = j < a.N;
        hist_add(h, ok ? a.cnt[j] >> 12 : 0u, ok);
    }
    __syncthreads();
    for (int i = tid; i < P_HB1; i += PT)
        if (h[i]) atomicAdd(&a.h1[i], h[i]);
}

// Level 2: the boundary bin b1 of level 1, then the histogram of count & 4095
// over the keys in it.
__global__ __launch_bounds__(PT) void k_prior_hist2(PriorArgs a)
{
    __shared__ uint32_t h[P_HB2];
    __shared__ uint32_t ws[PT / 64];
    __shared__ uint32_t s_res[2];
    const int tid = threadIdx.x;
    int b1;
    uint32_t above1;
    top_bin<P_HB1>(a.h1, 0u, (uint32_t)a.kk, ws, s_res, &b1, &above1);
    if (blockIdx.x == 0 && tid == 0) {
        a.par[0] = (uint32_t)b1;
        a.par[1] = above1;
    }
    for (int i = tid; i < P_HB2; i += PT) h[i] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * P_BLK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = base + (int64_t)i * PT + tid;
        const uint32_t v = j < a.N ? a.cnt[j] : 0u;
        const bool ok = j < a.N && (v >> 12) == (uint32_t)b1;
        hist_add(h, v & 4095u, ok);
    }
    __syncthreads();
    for (int i = tid; i < P_HB2; i += PT)
        if (h[i]) atomicAdd(&a.h2[i], h[i]);
}

// c* and the quota, then each block's counts above and at c*.
__global__ __launch_bounds__(PT) void k_prior_blocks(PriorArgs a)
{
    __shared__ uint32_t ws[PT / 64];
    __shared__ uint32_t s_res[2];
    const int tid = threadIdx.x;
    const uint32_t b1 = a.par[0], above1 = a.par[1];
    int b2;
    uint32_t gt;
    top_bin<P_HB2>(a.h2, above1, (uint32_t)a.kk, ws, s_res, &b2, &gt);
    const uint32_t cstar = (b1 << 12) | (uint32_t)b2;
    if (blockIdx.x == 0 && tid == 0) {
        a.par[2] = cstar;
        a.par[3] = gt;
        a.par[4] = (uint32_t)a.kk - gt;
    }
    const int64_t base = (int64_t)blockIdx.x * P_BLK + (int64_t)tid * 4;
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = base + i;
        if (j < a.N) {
            const uint32_t v = a.cnt[j];
            ngt += v > cstar ? 1u : 0u;
            neq += v == cstar ? 1u : 0u;
        }
    }
    uint32_t tgt, teq;
    block_excl_sum(ngt, ws, &tgt);
    block_excl_sum(neq, ws, &teq);
    if (tid == 0) {
        a.blk[2 * (size_t)blockIdx.x] = tgt;
        a.blk[2 * (size_t)blockIdx.x + 1] = teq;
    }
}

// Exclusive prefixes of the per-block counts (one workgroup, in place).
__global__ __launch_bounds__(PT) void k_prior_scan(PriorArgs a)
{
    __shared__ uint32_t ws[PT / 64];
    const int tid = threadIdx.x;
    uint32_t carry_gt = 0, carry_eq = 0;
    for (int b0 = 0; b0 < a.nblk; b0 += PT) {
        const int b = b0 + tid;
        const uint32_t g = b < a.nblk ? a.blk[2 * (size_t)b] : 0u;
        const uint32_t e = b < a.nblk ? a.blk[2 * (size_t)b + 1] : 0u;
        uint32_t tg, te;
        const uint32_t xg = block_excl_sum(g, ws, &tg);
        const uint32_t xe = block_excl_sum(e, ws, &te);
        if (b < a.nblk) {
            a.blk[2 * (size_t)b] = carry_gt + xg;
            a.blk[2 * (size_t)b + 1] = carry_eq + xe;
        }
        carry_gt += tg;
        carry_eq += te;
    }
}

// Writes every taken key at its rank in index order, and pads past k''.
__global__ __launch_bounds__(PT) void k_prior_emit(PriorArgs a)
{
    __shared__ uint32_t ws[PT / 64];
    const int tid = threadIdx.x;
    const uint32_t cstar = a.par[2], quota = a.par[4];
    const uint32_t gt0 = a.blk[2 * (size_t)blockIdx.x], eq0 = a.blk[2 * (size_t)blockIdx.x + 1];
    const int64_t base = (int64_t)blockIdx.x * P_BLK + (int64_t)tid * 4;
    uint32_t v[4], ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = base + i;
        v[i] = j < a.N ? a.cnt[j] : 0u;
        const bool ok = j < a.N;
        ngt += ok && v[i] > cstar ? 1u : 0u;
        neq += ok && v[i] == cstar ? 1u : 0u;
    }
    uint32_t tg, te;
    uint32_t gb = gt0 + block_excl_sum(ngt, ws, &tg);
    uint32_t eb = eq0 + block_excl_sum(neq, ws, &te);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = base + i;
        if (j < a.N) {
            if (v[i] > cstar) {
                a.out[gb + (eb < quota ? eb : quota)] = (int32_t)j;
                ++gb;
            } else if (v[i] == cstar) {
                if (eb < quota) a.out[gb + eb] = (int32_t)j;
                ++eb;
            }
        }
    }
    if (blockIdx.x == 0)
        for (int i = a.kk + tid; i < a.k_prime; i += PT) a.out[i] = -1;
}

}  // namespace

itk_status plan_prior(int32_t T_prev, int32_t k, int64_t N, int32_t k_prime, PriorPlan *out)
{
    if (T_prev < 0 || k <= 0 || N <= 0 || k_prime <= 0) return ITK_ERR_INVALID_ARG;
    if (N > (int64_t)0x7FFFFFFF) return ITK_ERR_UNSUPPORTED;
    if ((int64_t)T_prev * k > P_MAX_ENTRIES) return ITK_ERR_UNSUPPORTED;  // counts below 2^25
    PriorPlan p;
    p.N = N; p.T_prev = T_prev; p.k = k; p.k_prime = k_prime;
    p.nblk = (int32_t)((N + P_BLK - 1) / P_BLK);
    size_t off = 0;
    p.off_count = off; off = align256(off + (size_t)N * sizeof(uint32_t));
    p.off_h1 = off; off = align256(off + (size_t)P_HB1 * sizeof(uint32_t));
    p.off_h2 = off; off = align256(off + (size_t)P_HB2 * sizeof(uint32_t));
    p.off_blk = off; off = align256(off + (size_t)p.nblk * 2 * sizeof(uint32_t));
    p.off_par = off; off = align256(off + 8 * sizeof(uint32_t));
    p.bytes = off;
    *out = p;
    return ITK_OK;
}

hipError_t launch_prior(const PriorPlan &p, const int32_t *prev_idx, int32_t *prior_out, void *ws, hipStream_t stream)
{
    char *w = static_cast<char *>(ws);
    PriorArgs a;
    a.prev = prev_idx;
    a.n_entries = (int64_t)p.T_prev * p.k;
    a.cnt = reinterpret_cast<uint32_t *>(w + p.off_count);
    a.h1 = reinterpret_cast<uint32_t *>(w + p.off_h1);
    a.h2 = reinterpret_cast<uint32_t *>(w + p.off_h2);
    a.blk = reinterpret_cast<uint32_t *>(w + p.off_blk);
    a.par = reinterpret_cast<uint32_t *>(w + p.off_par);
    a.out = prior_out;
    a.N = p.N;
    a.k_prime = p.k_prime;
    a.kk = (int32_t)(p.k_prime < p.N ? p.k_prime : p.N);
    a.nblk = p.nblk;
    a.nrange = (int32_t)((p.N + P_RANGE - 1) / P_RANGE);
    const unsigned clear_blocks = (unsigned)std::max<int64_t>((p.N + PT - 1) / PT > 2048 ? 2048 : (p.N + PT - 1) / PT,
                                                              (P_HB1 + PT - 1) / PT);
    hipError_t e = launch_kernel(k_prior_clear, dim3(clear_blocks), dim3(PT), stream, a);
    if (e != hipSuccess) return e;
    const int64_t nslice = (a.n_entries + P_SLICE - 1) / P_SLICE;
    if (nslice > 0) {
        e = a.nrange <= P_MAX_RANGES
                ? launch_kernel(k_prior_count, dim3((unsigned)(a.nrange * nslice)), dim3(PT), stream, a)
                : launch_kernel(k_prior_count_direct,
                                dim3((unsigned)std::min<int64_t>((a.n_entries + PT - 1) / PT, 4096)), dim3(PT),
                                stream, a);
        if (e != hipSuccess) return e;
    }
    e = launch_kernel(k_prior_hist1, dim3((unsigned)p.nblk), dim3(PT), stream, a);
    if (e == hipSuccess) e = launch_kernel(k_prior_hist2, dim3((unsigned)p.nblk), dim3(PT), stream, a);
    if (e == hipSuccess) e = launch_kernel(k_prior_blocks, dim3((unsigned)p.nblk), dim3(PT), stream, a);
    if (e == hipSuccess) e = launch_kernel(k_prior_scan, dim3(1), dim3(PT), stream, a);
    if (e == hipSuccess) e = launch_kernel(k_prior_emit, dim3((unsigned)p.nblk), dim3(PT), stream, a);
    return e;
}

}  // namespace itk
