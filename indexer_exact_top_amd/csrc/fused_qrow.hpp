// Fused score + exact Top-k for single-head scoring (H == 1), e.g. inner-
// product retrieval (LiteTopK, arXiv 2607.11976, Sec. 3.1 Eq. (2)) or a
// one-head indexer (Sec. 2.1 Eq. (1) with H_I = 1).
//
// With one head per query, the head-rows mapping of fused_impl.hpp would fill
// one of the 32 MFMA rows.  Here the roles are turned around: the MFMA A
// operand is a block of 32 keys (rows, staged in LDS exactly as in the
// head-rows kernels), the B operand a block of 32 queries (columns, held in
// VGPRs), so every MFMA computes 32 x 32 useful scores.  A wave owns QROW_QB
// such query blocks, so each staged key fragment feeds QROW_QB MFMAs.  In the
// accumulator layout lane l holds query column l % 32 and 16 key rows, so a
// lane's per-query state (weight, length, gate) is one register per block.
//
// Steps (same method as the head-rows path, re-mapped):
//  * sample: the tile-strided view of every query is scored and stored
//    (bounded per query); one workgroup per query then places the gate at the
//    bin of the view's rank-q score, q = ceil(rho * k * n_view / L), with
//    m = 2048 equal-width bins over the view's range (the rank calibration of
//    the Sample-Guided paper, arXiv 2609.08450, Sec. 4.2);
//  * scan: every key of the query's range is scored, and a key is admitted
//    when its score is >= the query's gate; admitted keys go to a per-
//    (query, key split) slice, with slots from a per-wave LDS counter;
//  * select: one workgroup per query gathers its slices on chip and selects
//    exactly; a query whose slices overflowed or hold fewer than min(k, L)
//    candidates is re-scored and selected from its full row.
#pragma once

#include "fused_impl.hpp"

namespace itk {

#ifndef QROW_QBLOCKS
#define QROW_QBLOCKS 2
#endif
constexpr int QROW_QB = QROW_QBLOCKS;           // 32-query blocks per wave
constexpr int QROW_QPW = 32 * QROW_QB;          // queries per wave
constexpr int QROW_Q = QROW_QPW * FUSED_WAVES;  // queries per workgroup

// Without ReLU a score w * (q . k) is computed as |w| * ((sign(w) q) . k):
// negating the 16-bit query operands negates every product and partial sum
// exactly (round-to-nearest-even is symmetric), so the score is the same up to
// the sign of a zero (which the selection key ignores), and it becomes a
// non-decreasing function of the accumulator.  With ReLU nothing is folded.
template <class C>
__device__ __forceinline__ uint32_t qrow_qsign(float w)
{
    return (!C::RELU && (__float_as_uint(w) >> 31)) ? 0x80008000u : 0u;
}
template <class C>
__device__ __forceinline__ float qrow_weight(float w)
{
    return C::RELU ? w : __builtin_fabsf(w);
}

// Per-lane query state: lane l owns query column l % 32 of every block.
template <class C>
struct QRowQ {
    typename C::frag q[QROW_QB][C::KS];  // B fragments (8 values at k-slice l / 32)
    float w[QROW_QB];
    uint32_t L[QROW_QB];
    int t[QROW_QB];

    __device__ void load(const FusedArgs &a, int g)
    {
        const int l = (int)lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
        for (int qb = 0; qb < QROW_QB; ++qb) {
            t[qb] = g * QROW_Q + wave * QROW_QPW + qb * 32 + (l & 31);
            const bool act = t[qb] < a.T;
            const float wr = act ? a.W[t[qb]] : 0.f;
            const uint32_t sg = qrow_qsign<C>(wr);
            w[qb] = qrow_weight<C>(wr);
            L[qb] = act ? kv_length(a, t[qb]) : 0u;
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                const int d0 = kk * 16 + 8 * (l >> 5);
                const char *ptr = static_cast<const char *>(a.Q) + ((size_t)(act ? t[qb] : 0) * C::D + d0) * 2;
                const u32x4_t v = act ? *reinterpret_cast<const u32x4_t *>(ptr) : u32x4_t{0u, 0u, 0u, 0u};
                q[qb][kk] = u32x4_t{v[0] ^ sg, v[1] ^ sg, v[2] ^ sg, v[3] ^ sg};
            }
        }
    }

    __device__ __forceinline__ void settle()
    {
#pragma unroll
        for (int qb = 0; qb < QROW_QB; ++qb) {
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) asm volatile("" : "+v"(q[qb][kk]));
            asm volatile("" : "+v"(w[qb]));
        }
    }
};

// Score of one accumulator value: w * ReLU(q . k) (or w * q . k without
// ReLU), times the key's FP8 scale.  The same expression is used by every
// route, so a key's score does not depend on the route.
template <class C>
__device__ __forceinline__ float qrow_score(float acc, float w, float scale)
{
    float s = (C::RELU ? relu_bits(acc) : acc) * w;
    if constexpr (C::SCALE) s *= scale;
    return s;
}

// Key row held by accumulator register r of lane l, relative to the block.
__device__ __forceinline__ int qrow_key_of(int r, int l)
{
    return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
}

// MFMAs of one 32-key block: keys (A, from LDS at the lane's fragment address
// `al`) against the lane's query blocks (B, registers).
template <class C>
__device__ __forceinline__ void qrow_block_mfma(f32x16_t (&acc)[QROW_QB], const QRowQ<C> &qq, const char *al)
{
    constexpr int KCH = C::KS < 8 ? C::KS : (C::KS >= 16 ? 4 : 8);  // register budget at D = 256
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb) acc[qb] = f32x16_t{};
#pragma unroll
    for (int k0 = 0; k0 < C::KS; k0 += KCH) {
        typename C::frag a[KCH];
#pragma unroll
        for (int i = 0; i < KCH; ++i) a[i] = *reinterpret_cast<const u32x4_t *>(al + (k0 + i) * 32);
#pragma unroll
        for (int i = 0; i < KCH; ++i)
#pragma unroll
            for (int qb = 0; qb < QROW_QB; ++qb) acc[qb] = mfma32<C::MT>(a[i], qq.q[qb][k0 + i], acc[qb]);
    }
}

// Per-key FP8 scales of the 16 keys a lane holds in a block (4 groups of 4
// consecutive keys).
template <class C>
__device__ __forceinline__ void qrow_block_scales(float (&sc)[16], const float *tile_scale, int blk)
{
    const int l = (int)lane_id();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(tile_scale + blk * 32 + 8 * g + 4 * (l >> 5));
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[4 * g + j] = v[j];
    }
}

// 64-key tiles per stage of the main scan: copied keys take stages of about
// 64 KB per buffer (two buffers), so that each stage's copy has several
// microseconds of MFMA work to hide behind; FP8 keys move one tile per stage
// through registers.
template <class C>
constexpr int qrow_stage_tiles()
{
    return !C::DMA ? 1 : (C::ROWB <= 128 ? 8 : (C::ROWB <= 256 ? 4 : 2));
}

// The pipelined QRow scan: `nstages` stages of NSUB 64-key tiles, the first
// at key `first`, `step` keys apart, keys at or beyond `key_end` skipped.
// visit(kb0, acc, sc) is called once per computed 32-key block (wave-uniform)
// with the block's first key and the accumulators (and FP8 scales).  Every
// thread of the workgroup must call this.
template <class C, int NSUB, class Visit>
__device__ __forceinline__ void qrow_scan(const FusedArgs &a, TileBuf<C, NSUB> &tb, const QRowQ<C> &qq, int64_t first,
                                          int64_t step, int nstages, int64_t key_end, uint32_t wave_maxL,
                                          Visit &&visit)
{
    static_assert(C::DMA || NSUB == 1, "FP8 staging moves one 64-key tile per stage");
    static_assert(sizeof(tb.k[0]) == NSUB * C::TILE_LDS, "stage buffer size");
    const int64_t kend = key_end < (int64_t)wave_maxL ? key_end : (int64_t)wave_maxL;
    KStage<C> ks;
    DmaPlan<C, NSUB> dp;
    if constexpr (C::DMA) dp.init();
    if (nstages > 0) {
        if constexpr (C::DMA) {
            dp.issue(a, tb, 0, first);
        } else {
            ks.load(a, first);
            ks.store(tb, 0);
        }
    }
    const_cast<QRowQ<C> &>(qq).settle();
    wait_vmem_all();
    __syncthreads();
    const int boff = bfrag_lane_off<C>();
    for (int st = 0; st < nstages; ++st) {
        const int64_t skey = first + (int64_t)st * step;
        const int buf = st & 1;
        if (st + 1 < nstages) {
            if constexpr (C::DMA) dp.issue(a, tb, buf ^ 1, skey + step);
            else ks.load(a, skey + step);
        }
#pragma unroll
        for (int blk = 0; blk < 2 * NSUB; ++blk) {
            const int64_t kb0 = skey + blk * 32;
            if (kb0 < kend) {
                f32x16_t acc[QROW_QB];
                qrow_block_mfma<C>(acc, qq, tb.k[buf] + boff + blk * 32 * C::ROWP);
                float sc[16];
                if constexpr (C::SCALE) qrow_block_scales<C>(sc, tb.scale[buf], blk);
                visit(kb0, acc, sc);
            }
        }
        if (st + 1 < nstages) {
            if constexpr (!C::DMA) ks.store(tb, buf ^ 1);
            wait_vmem_all();
        }
        __syncthreads();
    }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0x111, 0xF>(v, 0u));
    v = max(v, dpp_u32<0x112, 0xF>(v, 0u));
    v = max(v, dpp_u32<0x114, 0xF>(v, 0u));
    v = max(v, dpp_u32<0x118, 0xF>(v, 0u));
    v = max(v, dpp_u32<0x142, 0xA>(v, 0u));
    v = max(v, dpp_u32<0x143, 0xC>(v, 0u));
    return lane_value(v, 63);
}

// ------------------------------------------------ sample: score the view
template <class C>
__global__ __launch_bounds__(FUSED_THREADS) void k_qrow_sample(FusedArgs a)
{
    __shared__ TileBuf<C, 1> tb;
    const int l = (int)lane_id();
    int g, p;
    map_group_split(blockIdx.x, a.G, a.Ps, g, p);
    QRowQ<C> qq;
    qq.load(a, g);
    const uint32_t wave_maxL = wave_max_u32(max(qq.L[0], qq.L[QROW_QB - 1]));
    uint32_t gmaxL = 0;  // the view of the workgroup's longest query
    {
        __shared__ uint32_t s_max;
        if (threadIdx.x == 0) s_max = 0;
        __syncthreads();
        if (l == 0) atomicMax(&s_max, wave_maxL);
        __syncthreads();
        gmaxL = s_max;
    }
    const SampleIter it = sample_iter(a, g, p, gmaxL);
    const int64_t st = a.sample_tiles;
    const int64_t phase = g % a.sample_tiles;
    qrow_scan<C, 1>(a, tb, qq, it.first_key, it.stride_keys, it.ntiles, it.end, gmaxL,
                    [&](int64_t kb0, const f32x16_t (&acc)[QROW_QB], const float (&sc)[16]) {
                        // view position of key kb0: sampled tile ordinal * 64 + offset
                        const int64_t tile = kb0 / TILE_KEYS;
                        const int64_t vpos0 = ((tile - phase) / st) * TILE_KEYS + (kb0 - tile * TILE_KEYS);
#pragma unroll
                        for (int qb = 0; qb < QROW_QB; ++qb) {
                            if (qq.t[qb] >= a.T) continue;
                            float *row = a.samp + (size_t)qq.t[qb] * a.samp_cap;
                            if (kb0 + 32 <= (int64_t)qq.L[qb]) {
                                // registers 4g..4g+3 hold 4 consecutive keys: one 16-byte store each
#pragma unroll
                                for (int g4 = 0; g4 < 4; ++g4) {
                                    f32x4_t v;
#pragma unroll
                                    for (int j = 0; j < 4; ++j)
                                        v[j] = qrow_score<C>(acc[qb][4 * g4 + j], qq.w[qb], sc[4 * g4 + j]);
                                    *reinterpret_cast<f32x4_t *>(row + vpos0 + qrow_key_of(4 * g4, l)) = v;
                                }
                            } else {
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int kr = qrow_key_of(r, l);
                                    if (kb0 + kr < (int64_t)qq.L[qb])
                                        row[vpos0 + kr] = qrow_score<C>(acc[qb][r], qq.w[qb], sc[r]);
                                }
                            }
                        }
                    });
}

// ------------------------------- gate: one workgroup per query, from the view
template <class C>
__global__ __launch_bounds__(SEL_THREADS) void k_qrow_gate(FusedArgs a)
{
    constexpr int NT = SEL_THREADS;
    __shared__ uint32_t hist[NBINS];
    __shared__ uint32_t scan[16];
    __shared__ float red[2][16];
    __shared__ BoundaryOut bo;
    const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t L = kv_length(a, t);
    const int g = t / QROW_Q;
    const RowSample rs = row_sample(a, t, g, L, false);
    // per-call reset of the query's slice counters
    for (int p = tid; p < 2 * a.P; p += NT) a.qcnt[(size_t)t * a.P * 2 + p] = 0u;
    if (rs.admit_all) {
        if (tid == 0) a.gate[t] = -__builtin_inff();
        return;
    }
    const float *row = a.samp + (size_t)t * a.samp_cap;
    const uint32_t n = rs.n_a;
    // A view of at most VR * NT scores is loaded once, all of a thread's
    // loads in flight together, and kept in registers for both passes.
    constexpr int VR = 32;
    const bool resident = n <= (uint32_t)(VR * NT);
    float vr[VR];
    float mn = __builtin_inff(), mx = -__builtin_inff();
    if (resident) {
#pragma unroll
        for (int j = 0; j < VR; ++j) {
            const uint32_t i = tid + j * NT;
            vr[j] = i < n ? row[i] : __builtin_nanf("");
        }
#pragma unroll
        for (int j = 0; j < VR; ++j) {
            mn = fminf(mn, vr[j]);
            mx = fmaxf(mx, vr[j]);
        }
    } else {
        for (uint32_t i0 = tid; i0 < n; i0 += 8 * NT) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t i = i0 + j * NT;
                v[j] = i < n ? row[i] : __builtin_nanf("");
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                mn = fminf(mn, v[j]);
                mx = fmaxf(mx, v[j]);
            }
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = mx;
    }
    for (int i = tid; i < NBINS; i += NT) hist[i] = 0u;
    __syncthreads();
    mn = red[0][0];
    mx = red[1][0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        mn = fminf(mn, red[0][w]);
        mx = fmaxf(mx, red[1][w]);
    }
    const float scale = (float)NBINS / (mx - mn);
    if (!(mx > mn) || !__builtin_isfinite(scale) || !(scale > 0.f) || !__builtin_isfinite(mn)) {
        if (tid == 0) a.gate[t] = -__builtin_inff();
        return;
    }
    auto bin_add = [&](float v) {
        if (v == v) atomicAdd(&hist[(uint32_t)fminf(fmaxf(floorf((v - mn) * scale), 0.f), (float)(NBINS - 1))], 1u);
    };
    if (resident) {
#pragma unroll
        for (int j = 0; j < VR; ++j) bin_add(vr[j]);
    } else {
        for (uint32_t i0 = tid; i0 < n; i0 += 8 * NT) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t i = i0 + j * NT;
                v[j] = i < n ? row[i] : __builtin_nanf("");
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) bin_add(v[j]);
        }
    }
    __syncthreads();
    find_boundary<NT>(hist, rs.q0, scan, &bo);
    if (tid == 0) {
        // every view score in bins >= the boundary bin is >= this value
        const float edge = bo.digit ? mn + (float)bo.digit / scale : -__builtin_inff();
        a.gate[t] = bo.digit ? fminf(edge, mx) : -__builtin_inff();
    }
}

// ------------------------------------------------ scan: gate and collect
// A value no larger than any accumulator whose score (qrow_score without
// per-key scales, weight w after folding) can reach `gate`: the scan tests the
// accumulator against it and computes the exact score only for the few that
// are not below it.  Scores are non-decreasing in the accumulator for w >= 0;
// for w < 0 (ReLU only) every accumulator is tested exactly.
__device__ __forceinline__ float qrow_acc_floor(float gate, float w, bool relu)
{
    const float ninf = -__builtin_inff();
    if (!(gate > ninf)) return ninf;
    if (w != w) return __builtin_nanf("");  // every score is NaN: nothing passes
    if (w < 0.f) return ninf;
    if (w == 0.f) return gate <= 0.f ? ninf : __builtin_inff();
    if (relu && gate <= 0.f) return ninf;
    // x * w >= gate (rounded) needs x >= gate / w up to about one ulp of each
    // rounding; 8 ulps below the quotient is safely below that.
    const float x = gate / w;
    if (x != x) return ninf;
    uint32_t u = __float_as_uint(x);
    uint32_t o = (u >> 31) ? ~u : (u | 0x80000000u);  // ascending order
    const uint32_t o_ninf = 0x007FFFFFu;               // order key of -inf
    o = o > o_ninf + 8u ? o - 8u : o_ninf;
    u = (o >> 31) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Appends every score of a 32-key block that is at or above the lane's gate
// to the lane's half of its (query, split) slice.  A block almost never has
// a passing score in a given accumulator register across the whole wave, so
// each register costs one multiply, one compare and one wave-uniform branch.
// Past the slice capacity the last slot is overwritten: the count still
// grows, and a count above the capacity sends the query to recovery.
template <class C, bool PARTIAL>
__device__ __forceinline__ void qrow_collect(const f32x16_t (&acc)[QROW_QB], const float (&sc)[16],
                                             const QRowQ<C> &qq, const float (&gate)[QROW_QB],
                                             const float (&afloor)[QROW_QB],
                                             const int64_t (&kend)[QROW_QB], int64_t kb0, Cand *const (&slice)[QROW_QB],
                                             uint32_t (&cnt)[QROW_QB], uint32_t capH)
{
    const int l = (int)lane_id();
    const uint32_t kb = (uint32_t)kb0 + 4u * (uint32_t)(l >> 5);  // key of register 0
    int32_t lim[QROW_QB];  // valid rows of the block (PARTIAL only): row < lim
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb) {
        const int64_t d = kend[qb] - kb0;
        lim[qb] = d < 0 ? 0 : (d > 32 ? 32 : (int32_t)d);
    }
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            bool maybe;
            if constexpr (C::SCALE) maybe = true;
            else maybe = acc[qb][r] >= afloor[qb];
            if (maybe) {
                const float s = qrow_score<C>(acc[qb][r], qq.w[qb], sc[r]);
                bool pass = s >= gate[qb];
                if constexpr (PARTIAL) pass = pass && qrow_key_of(r, l) < lim[qb];
                if (pass) {
                    const uint32_t slot = cnt[qb] < capH ? cnt[qb] : capH - 1u;
                    slice[qb][slot] = Cand{kb + (uint32_t)(8 * (r >> 2) + (r & 3)), s};
                    ++cnt[qb];
                }
            }
        }
}

template <class C>
__global__ __launch_bounds__(FUSED_THREADS) void k_qrow_main(FusedArgs a)
{
    __shared__ TileBuf<C, qrow_stage_tiles<C>()> tb;
    const int tid = threadIdx.x, l = tid & 63;
    int g, p;
    map_group_split(blockIdx.x, a.G, a.P, g, p);
    if (a.force == 1) return;  // every query takes the re-scoring route
    QRowQ<C> qq;
    qq.load(a, g);
    float gate[QROW_QB], afloor[QROW_QB];
    int64_t kend[QROW_QB];
    const int64_t k_lo = (int64_t)p * a.span;
    int64_t k_hi = k_lo + a.span;
    uint32_t wmax = 0;
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb) {
        const bool act = qq.t[qb] < a.T;
        gate[qb] = act ? a.gate[qq.t[qb]] : __builtin_inff();
        afloor[qb] = qrow_acc_floor(gate[qb], qq.w[qb], C::RELU);
        kend[qb] = (int64_t)qq.L[qb] < k_hi ? (int64_t)qq.L[qb] : k_hi;
        wmax = max(wmax, qq.L[qb]);
    }
    __shared__ uint32_t s_max;
    if (tid == 0) s_max = 0;
    __syncthreads();
    wmax = wave_max_u32(wmax);
    if (l == 0) atomicMax(&s_max, wmax);
    __syncthreads();
    const uint32_t gmaxL = s_max;
    if (k_hi > (int64_t)gmaxL) k_hi = gmaxL;
    constexpr int SK = qrow_stage_tiles<C>() * TILE_KEYS;  // keys per stage
    const int nstages = k_hi > k_lo ? (int)((k_hi - k_lo + SK - 1) / SK) : 0;
    // keys below kmin are valid for every lane's queries (wave-uniform)
    uint32_t kmin_l = 0xFFFFFFFFu;
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb)
        kmin_l = min(kmin_l, (uint32_t)(kend[qb] > k_lo ? kend[qb] - k_lo : 0));
    const uint32_t kmin = ~wave_max_u32(~kmin_l);  // wave minimum
    // Each lane appends to its own half of the (query, split) slice, with a
    // register counter: lanes l and l + 32 hold different keys of the same
    // query, so their halves never collide and no atomics are needed.
    const uint32_t capH = (uint32_t)a.capS / 2u;
    const int h = l >> 5;
    Cand *myslice[QROW_QB];
    uint32_t cnt[QROW_QB];
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb) {
        const int tq = qq.t[qb] < a.T ? qq.t[qb] : 0;
        myslice[qb] = a.cand + (((size_t)tq * a.P + p) * 2 + h) * capH;
        cnt[qb] = 0;
    }

    qrow_scan<C, qrow_stage_tiles<C>()>(a, tb, qq, k_lo, SK, nstages, k_hi, gmaxL,
                          [&](int64_t kb0, const f32x16_t (&acc)[QROW_QB], const float (&sc)[16]) {
                              // Block entirely below every query's length: no
                              // per-key validity test (wave-uniform choice).
                              if (kb0 + 32 <= k_lo + (int64_t)kmin)
                                  qrow_collect<C, false>(acc, sc, qq, gate, afloor, kend, kb0, myslice, cnt, capH);
                              else
                                  qrow_collect<C, true>(acc, sc, qq, gate, afloor, kend, kb0, myslice, cnt, capH);
                          });
#pragma unroll
    for (int qb = 0; qb < QROW_QB; ++qb)
        if (qq.t[qb] < a.T) a.qcnt[((size_t)qq.t[qb] * a.P + p) * 2 + h] = cnt[qb];
}

// --------------------------------------- select, and re-scoring per query
// Every valid key of query t, re-scored with the same operand layout as the
// scan (the query in column 0 of the B operand, 32 keys per MFMA as rows), so
// that every score equals the scan's.  Lanes 0 and 32 hold the results.
template <class C>
struct QRowRescoreSrc {
    const FusedArgs *a;
    int t;
    uint32_t L;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        const int l = (int)lane_id();
        const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
        const float wr = a->W[t];
        const uint32_t sg = qrow_qsign<C>(wr);
        const float w = qrow_weight<C>(wr);
        typename C::frag qf[C::KS];
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            const int d0 = kk * 16 + 8 * (l >> 5);
            const u32x4_t v = (l & 31) == 0 ? *reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a->Q) +
                                                                                 ((size_t)t * C::D + d0) * 2)
                                            : u32x4_t{0u, 0u, 0u, 0u};
            qf[kk] = u32x4_t{v[0] ^ sg, v[1] ^ sg, v[2] ^ sg, v[3] ^ sg};
        }
        for (int64_t kb0 = (int64_t)wave * 32; kb0 < (int64_t)L; kb0 += (int64_t)nw * 32) {
            const int64_t key = kb0 + (l & 31);
            const bool ok = key < a->N;
            const char *krow = static_cast<const char *>(a->K) + (size_t)(ok ? key : 0) * C::D * C::kbytes;
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                const int d0 = kk * 16 + 8 * (l >> 5);
                u32x4_t af;
                if constexpr (C::KT == ITK_FP8_E4M3) {
                    const u32x2_t raw = ok ? *reinterpret_cast<const u32x2_t *>(krow + d0) : u32x2_t{0u, 0u};
                    const u32x2_t lo = fp8x4_widen<C::MT>(raw[0]), hi = fp8x4_widen<C::MT>(raw[1]);
                    af = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    af = ok ? *reinterpret_cast<const u32x4_t *>(krow + d0 * 2) : u32x4_t{0u, 0u, 0u, 0u};
                }
                acc = mfma32<C::MT>(af, qf[kk], acc);
            }
            if ((l & 31) == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t kr = kb0 + qrow_key_of(r, l);
                    if (kr < (int64_t)L) {
                        const float sc = C::SCALE ? a->k_scale[kr] : 1.f;
                        f((uint32_t)kr, qrow_score<C>(acc[r], w, sc));
                    }
                }
            }
        }
    }
};

// Items of a query's candidate slices (prefix offsets in cpre), streamed.
struct QRowSliceSrc {
    const Cand *slices;  // [P][capS]
    const uint32_t *cpre;
    int P;
    uint32_t capS;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        for (int c = 0; c < P; ++c) {
            const uint32_t n = cpre[c + 1] - cpre[c];
            const Cand *s = slices + (size_t)c * capS;
            for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
                const Cand e = s[i];
                f(e.idx, e.val);
            }
        }
    }
};

constexpr int QROW_STASH = 16384;  // candidates kept on chip by the single-head select
constexpr int QROW_RESCORE_THREADS = 512;

template <class C>
__global__ __launch_bounds__(SEL_THREADS) void k_qrow_select(FusedArgs a)
{
    constexpr int NT = SEL_THREADS;
    __shared__ SelectSmemT<QROW_STASH> sm;
    static_assert(2 * QROW_MAX_SPLITS <= NT, "one slice per thread in the count prefix");
    __shared__ uint32_t cpre[2 * QROW_MAX_SPLITS + 1];
    __shared__ uint32_t s_ovf;
    __shared__ uint32_t s_wsum[NT / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x;
    const uint32_t L = kv_length(a, t);
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    const int ncell = 2 * a.P;                 // (split, half) slices of the query
    const uint32_t capH = (uint32_t)a.capS / 2u;
    int32_t *oi = a.out_idx + (size_t)t * a.k;
    float *os = a.out_score + (size_t)t * a.k;
    for (uint32_t i = need + tid; i < (uint32_t)a.k; i += NT) {
        oi[i] = -1;
        os[i] = -__builtin_inff();
    }
    if (need == 0) {
        if (tid == 0 && a.route) a.route[t] = 4;
        if (tid == 0 && a.count) a.count[t] = 0;
        if (tid == 0) a.rflag[t] = 0u;
        return;
    }
    // slice counts -> prefix (cpre) and overflow flag: one slice per thread,
    // all counts loaded at once, then a block-wide prefix sum
    if (tid == 0) s_ovf = 0;
    const uint32_t *cnt = a.qcnt + (size_t)t * ncell;
    const uint32_t raw = tid < ncell ? cnt[tid] : 0u;
    __syncthreads();
    if (raw > capH) atomicOr(&s_ovf, 1u);
    const uint32_t incl = wave_incl_sum(min(raw, capH));
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    {
        uint32_t off = 0;
        for (int w = 0; w < wave; ++w) off += s_wsum[w];
        if (tid < ncell) cpre[tid + 1] = off + incl;
        if (tid == 0) cpre[0] = 0;
    }
    __syncthreads();
    const uint32_t n = cpre[ncell];
    // a query whose slices overflowed or hold fewer than min(k, L)
    // candidates is left to k_qrow_rescore
    const bool recover = a.force == 1 || s_ovf || n < need;
    if (tid == 0) a.rflag[t] = recover ? 1u : 0u;
    if (tid == 0 && a.count) {  // admitted candidates, past the slices' capacity included
        uint32_t tot = 0;
        for (int c = 0; c < ncell; ++c) tot += cnt[c];
        a.count[t] = (int32_t)tot;
    }
    auto emit = [&](uint32_t slot, uint64_t K) {
        if (slot < need) {
            oi[slot] = (int32_t)key_index(K);
            os[slot] = key_value(K);
        }
    };
    if (!recover && n <= (uint32_t)QROW_STASH) {
        // Gather: item i of the query's n candidates lives in the slice c with
        // cpre[c] <= i < cpre[c + 1] (binary search in LDS), so every thread
        // has B independent loads in flight whatever the slices' sizes.  The
        // value range is taken on the way.
        constexpr int B = 8;
        const Cand *base = a.cand + (size_t)t * ncell * capH;
        float mn = __builtin_inff(), mx = -__builtin_inff();
        for (uint32_t i0 = tid; i0 < n; i0 += B * NT) {
            Cand e[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint32_t i = i0 + j * NT;
                if (i < n) {
                    // largest lo < ncell with cpre[lo] <= i, in a fixed number
                    // of steps, so that the B searches of a thread interleave
                    // (every index read stays below 2 * QROW_MAX_SPLITS)
                    int lo = 0;
#pragma unroll
                    for (int step = QROW_MAX_SPLITS; step >= 1; step >>= 1)
                        if (lo + step < ncell && cpre[lo + step] <= i) lo += step;
                    e[j] = base[(size_t)lo * capH + (i - cpre[lo])];
                }
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint32_t i = i0 + j * NT;
                if (i < n) {
                    sm.stash[i] = make_key(e[j].val, e[j].idx);
                    mn = fminf(mn, e[j].val);
                    mx = fmaxf(mx, e[j].val);
                }
            }
        }
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane == 0) {
            sm.vmin[wave] = mn;
            sm.vmax[wave] = mx;
        }
        __syncthreads();
        select_stashed<NT>(sm, n, need, emit, true);
    } else if (!recover) {
        QRowSliceSrc src{a.cand + (size_t)t * ncell * capH, cpre, ncell, capH};
        exact_select<NT>(sm, src, need, emit);
    }
    if (tid == 0 && a.route) a.route[t] = recover ? 3 : 1;
}

// The re-scoring route of the single-head selection, for the queries that
// k_qrow_select flagged: every valid key of the query is re-scored from Q
// and K (QRowRescoreSrc, the scan's operand layout, so the scores equal the
// scan's) and the query is selected exactly by one workgroup.  A kernel of
// its own, so that the selection does not carry the re-scoring registers on
// every query (they made it spill), with 512 threads, whose register budget
// holds the re-scoring without spills.  RESCORE_GROUPS workgroups share the
// queries (workgroup b takes queries b, b + gridDim.x, ...) and check them a
// chunk of one query per thread at a time, with one vote, so that a call
// with no flagged query costs about one memory round trip.
template <class C>
__global__ __launch_bounds__(QROW_RESCORE_THREADS) void k_qrow_rescore(FusedArgs a)
{
    __shared__ SelectSmemT<QROW_STASH> sm;
    for (int base = 0; blockIdx.x + (int64_t)base * gridDim.x < a.T; base += QROW_RESCORE_THREADS) {
        const int64_t ti = blockIdx.x + (int64_t)(base + threadIdx.x) * gridDim.x;
        if (!__syncthreads_or(ti < a.T && a.rflag[ti] != 0u)) continue;
        for (int j = 0; j < QROW_RESCORE_THREADS; ++j) {
            const int64_t tj = blockIdx.x + (int64_t)(base + j) * gridDim.x;
            if (tj >= a.T) break;
            const int t = (int)tj;
            if (!a.rflag[t]) continue;  // workgroup-uniform
            const uint32_t L = kv_length(a, t);
            const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
            int32_t *oi = a.out_idx + (size_t)t * a.k;
            float *os = a.out_score + (size_t)t * a.k;
            auto emit = [&](uint32_t slot, uint64_t K) {
                if (slot < need) {
                    oi[slot] = (int32_t)key_index(K);
                    os[slot] = key_value(K);
                }
            };
            QRowRescoreSrc<C> src{&a, t, L};
            exact_select<QROW_RESCORE_THREADS>(sm, src, need, emit);
            __syncthreads();  // the next query reuses sm
        }
    }
}

// --------------------------------------------------------------- launch
template <class C>
hipError_t launch_qrow_cfg(const FusedPlan &p, const FusedArgs &a, hipStream_t stream)
{
    hipError_t e;
    {
        StageTimer st(ST_F_MINMAX, stream);
        e = launch_kernel(k_qrow_sample<C>, dim3(p.G * p.Ps), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_HIST, stream);
        e = launch_kernel(k_qrow_gate<C>, dim3(p.T), dim3(SEL_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_MAIN, stream);
        e = launch_kernel(k_qrow_main<C>, dim3(p.G * p.P), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_SELECT, stream);
        e = launch_kernel(k_qrow_select<C>, dim3(p.T), dim3(SEL_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_RESCORE, stream);
        e = launch_kernel(k_qrow_rescore<C>, dim3(p.T < RESCORE_GROUPS ? p.T : RESCORE_GROUPS), dim3(QROW_RESCORE_THREADS),
                          stream, a);
    }
    return e;
}

FusedLauncher find_qrow_launcher(int qt, int kt, int d, bool relu);

#define ITK_QROW_CASES_FOR(QT, KT)                                                                       \
    if (qt == QT && kt == KT) {                                                                          \
        if (d == 64) return relu ? &launch_qrow_cfg<FCfg<QT, KT, 1, 64, true>>                           \
                                 : &launch_qrow_cfg<FCfg<QT, KT, 1, 64, false>>;                         \
        if (d == 128) return relu ? &launch_qrow_cfg<FCfg<QT, KT, 1, 128, true>>                         \
                                  : &launch_qrow_cfg<FCfg<QT, KT, 1, 128, false>>;                       \
        if (d == 256) return relu ? &launch_qrow_cfg<FCfg<QT, KT, 1, 256, true>>                         \
                                  : &launch_qrow_cfg<FCfg<QT, KT, 1, 256, false>>;                       \
    }

}  // namespace itk
