// Device building blocks shared by the standalone and the fused Top-k.
//
//  * ordered fp32 keys and the 64-bit composite key (value, inverted index)
//    whose descending order is "score descending, index ascending";
//  * the 11-bit coarse key of the sampled view (Sample-Guided Exact Top-K,
//    Sec. 4.2: the fp16 ordered key shifted right by 5, 2^11 bins) and the
//    inclusive fp32 endpoint of a coarse bin (Sec. 5.2);
//  * a block-wide boundary search over a 2048-bin LDS histogram;
//  * select_stashed: a value histogram over candidates held in LDS commits
//    every bin above the boundary bin and leaves only that bin to settle;
//  * exact_select: frontier radix refinement over the composite key.  Digits
//    11+11+10 of the ordered fp32 key resolve the value (Sec. 5.4); three more
//    digits of the inverted index resolve the final equal-value group in favour
//    of the lower indices.  Every round commits the strictly better digit
//    groups and retains only the boundary group (Sec. 4.4 commit/retain).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace itk {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a CDNA buffer resource for raw (untyped) dword accesses: 32-bit
// data format, no swizzle.  Accesses past the resource's byte range are
// dropped (stores) or return zero (loads).
constexpr int BUF_RSRC_WORD3 = 0x00020000;

constexpr int NBINS = 2048;       // one 2^11-bin histogram, reused by every round
constexpr int STASH_CAP = 7680;   // items kept on chip (60 KB of composite keys)
constexpr int BOUND_CAP = 1024;   // boundary-bin items kept for the final exact rounds
constexpr int RANK_CAP = 128;     // boundary bins up to this size are settled by ranking

// ----------------------------------------------------------------- keys
// Order-preserving map fp32 -> u32 (larger value -> larger key).  -0 is
// mapped like +0 so that equal values get equal keys.
__device__ __forceinline__ uint32_t ordered_key(float x)
{
    uint32_t b = __float_as_uint(x);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_key(uint32_t u)
{
    const uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(b);
}

// Composite key: descending order == (value desc, index asc); unique per index.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx)
{
    return ((uint64_t)ordered_key(v) << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t K) { return ~(uint32_t)K; }
__device__ __forceinline__ float key_value(uint64_t K) { return from_ordered_key((uint32_t)(K >> 32)); }

// Radix levels over the composite key: 11+11+10 value bits, then 11+11+10
// bits of the inverted index.
__device__ __forceinline__ int level_shift(int l)
{
    return l == 0 ? 53 : l == 1 ? 42 : l == 2 ? 32 : l == 3 ? 21 : l == 4 ? 10 : 0;
}
__device__ __forceinline__ int level_width(int l) { return (l == 2 || l == 5) ? 10 : 11; }
__device__ __forceinline__ uint32_t key_digit(int l, uint64_t K)
{
    return (uint32_t)(K >> level_shift(l)) & ((1u << level_width(l)) - 1u);
}
__device__ __forceinline__ uint64_t level_mask(int l)
{
    return (uint64_t)((1u << level_width(l)) - 1u) << level_shift(l);
}

// 11-bit coarse key: fp16 (round to nearest even) ordered key >> 5.
// Monotone non-decreasing in x.
__device__ __forceinline__ uint32_t coarse_key(float x)
{
    const float xc = (__float_as_uint(x) == 0x80000000u) ? 0.0f : x;
    const _Float16 h = (_Float16)xc;
    const uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
    const uint32_t o = (hb & 0x8000u) ? (~hb & 0xFFFFu) : (hb | 0x8000u);
    return o >> 5;
}

__device__ __forceinline__ uint32_t lane_id_early() { return __lane_id(); }

// Smallest fp32 value x (over [-inf, +inf]) with coarse_key(x) >= tau: then
// "x >= endpoint" reproduces "coarse_key(x) >= tau" with one compare.  Bins
// above the bin of +inf hold only NaN codes; their endpoint is NaN, which
// admits no value.  Searched by one whole wave: every round splits the open
// interval (lo, hi] of ordered keys into 64 parts, each lane tests one split
// point, and the lowest passing part becomes the new interval (coarse_key is
// monotone, so the predicate is a step function of the ordered key).  Six
// rounds resolve 32 bits.  All lanes of the wave must call it; every lane
// gets the result.
__device__ inline float coarse_endpoint_wave(uint32_t tau)
{
    uint32_t lo = ordered_key(-__builtin_inff());
    uint32_t hi = ordered_key(__builtin_inff());
    if (coarse_key(from_ordered_key(lo)) >= tau) return -__builtin_inff();
    if (coarse_key(from_ordered_key(hi)) < tau) return __builtin_nanf("");
    const uint32_t l = lane_id_early();
    while (hi - lo > 1u) {  // coarse(lo) < tau <= coarse(hi)
        const uint64_t span = (uint64_t)(hi - lo);
        // split points lo + span*(l+1)/64 for l = 0..62 (lane 63 is hi itself)
        const uint32_t pt = l < 63u ? lo + (uint32_t)((span * (l + 1u)) >> 6) : hi;
        const bool ok = pt > lo && coarse_key(from_ordered_key(pt)) >= tau;
        const uint64_t m = __ballot(ok);            // lane 63 always passes
        const int f = __ffsll((unsigned long long)m) - 1;
        const uint32_t new_hi = (uint32_t)__builtin_amdgcn_readlane((int)pt, f);
        uint32_t new_lo = (uint32_t)__builtin_amdgcn_readlane((int)pt, f > 0 ? f - 1 : 0);
        if (f == 0 || new_lo <= lo) new_lo = lo;
        lo = new_lo;
        hi = new_hi;
    }
    return from_ordered_key(hi);
}

// ---------------------------------------------------------- wave helpers
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Cross-lane steps in registers (DPP), not through LDS: row_shr:n moves each
// lane's value n lanes up within its row of 16, row_bcast:15 / row_bcast:31
// hand lane 15 / 31 to the following rows.  Lanes without a source take
// `identity`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: lane l gets sum_{l' <= l} v.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v)
{
    v += dpp_u32<0x111, 0xF>(v, 0u);  // row_shr:1
    v += dpp_u32<0x112, 0xF>(v, 0u);  // row_shr:2
    v += dpp_u32<0x114, 0xF>(v, 0u);  // row_shr:4
    v += dpp_u32<0x118, 0xF>(v, 0u);  // row_shr:8
    v += dpp_u32<0x142, 0xA>(v, 0u);  // row_bcast:15 into rows 1, 3
    v += dpp_u32<0x143, 0xC>(v, 0u);  // row_bcast:31 into rows 2, 3
    return v;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Inclusive suffix sum over the lanes of a wave: lane l gets sum_{l' >= l} v.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v)
{
    const uint32_t incl = wave_incl_sum(v);
    return lane_value(incl, 63) - incl + v;
}

// Wave-wide min / max of a float (every lane gets the result).
__device__ __forceinline__ float wave_min(float x)
{
    const uint32_t inf = __float_as_uint(__builtin_inff());
    uint32_t v = __float_as_uint(x);
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x111, 0xF>(v, inf))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x112, 0xF>(v, inf))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x114, 0xF>(v, inf))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x118, 0xF>(v, inf))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x142, 0xA>(v, inf))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(dpp_u32<0x143, 0xC>(v, inf))));
    return __uint_as_float(lane_value(v, 63));
}
__device__ __forceinline__ float wave_max(float x) { return -wave_min(-x); }

// Reserve `count` consecutive slots per lane from an LDS or global counter
// with one atomic per wave; returns the lane's first slot.  Every lane of the
// wave must call it (count may be 0).
__device__ __forceinline__ uint32_t wave_reserve_n(uint32_t count, uint32_t *ctr)
{
    const uint32_t incl = wave_incl_sum(count);
    const uint32_t total = lane_value(incl, 63);
    uint32_t base = 0;
    if (total) {
        if (lane_id() == 0u) base = atomicAdd(ctr, total);
        base = lane_value(base, 0);
    }
    return base + incl - count;
}

// Reserve one slot per active lane with `pred` from an LDS or global counter,
// with one atomic per wave.  Must be reached by every active lane.
__device__ __forceinline__ uint32_t wave_reserve(bool pred, uint32_t *ctr)
{
    const uint64_t m = __ballot(pred);
    uint32_t base = 0;
    if (m) {
        const int leader = __ffsll((unsigned long long)m) - 1;
        if ((int)lane_id() == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
        base = lane_value(base, leader);
    }
    return base + lanes_below(m);
}

// ------------------------------------------------- block boundary search
struct BoundaryOut {
    uint32_t digit;  // boundary bin
    uint32_t above;  // items in bins > digit
    uint32_t eq;     // items in the boundary bin
    uint32_t total;  // items in all bins
};

// d = max{b : sum_{b' >= b} hist[b'] >= quota}, for NQ quotas at once (one
// pass over the histogram).  When a quota exceeds the total, d = 0 and
// above + eq == total.  Block of NT threads; `scan` holds NT/64 words; `out`
// is an array of NQ results in LDS.  Ends with a barrier; the results are in
// `out` for every thread.
template <int NT, int NQ>
__device__ void find_boundaries(const uint32_t *hist, const uint32_t (&quota)[NQ], uint32_t *scan, BoundaryOut *out)
{
    constexpr int PER = NBINS / NT;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    uint32_t loc[PER];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        loc[i] = hist[tid * PER + i];
        s += loc[i];
    }
    const uint32_t incl = wave_suffix_sum(s);
    if (lane_id() == 0) scan[wave] = incl;
    __syncthreads();
    uint32_t above_waves = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        total += scan[w];
        if (w > wave) above_waves += scan[w];
    }
    const uint32_t excl = incl - s + above_waves;  // items in bins above this thread's bins
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (tid == 0 && total < quota[q]) {
            out[q].digit = 0;
            out[q].above = total - hist[0];
            out[q].eq = hist[0];
            out[q].total = total;
        }
        if (excl < quota[q] && excl + s >= quota[q]) {
            uint32_t cum = excl;
#pragma unroll
            for (int i = PER - 1; i >= 0; --i) {
                if (cum + loc[i] >= quota[q]) {
                    out[q].digit = (uint32_t)(tid * PER + i);
                    out[q].above = cum;
                    out[q].eq = loc[i];
                    out[q].total = total;
                    break;
                }
                cum += loc[i];
            }
        }
    }
    __syncthreads();
}

template <int NT>
__device__ void find_boundary(const uint32_t *hist, uint32_t quota, uint32_t *scan, BoundaryOut *out)
{
    const uint32_t q[1] = {quota};
    find_boundaries<NT, 1>(hist, q, scan, out);
}

// --------------------------------------------------------- exact select
// LDS of one selecting workgroup; CAP composite keys fit on chip.
template <int CAP>
struct SelectSmemT {
    static constexpr int cap = CAP;
    uint32_t hist[NBINS];
    uint64_t stash[CAP];
    uint64_t bound[BOUND_CAP];
    float vmin[16], vmax[16];
    uint32_t n_bound;
    uint64_t P, M;        // resolved prefix and its mask
    uint32_t quota;       // items still to take from the current region
    uint32_t level;
    uint32_t done, stashed, stash_n, out_n;
    BoundaryOut b;
    uint32_t scan[16];
};
using SelectSmem = SelectSmemT<STASH_CAP>;

// Exact Top-`need` of the items produced by `src` under the composite key.
//
// `src.for_each(f)` must call f(index, value) exactly once per item, spread
// over the threads of the block (every thread must call for_each; it may
// contain barriers).  `emit(slot, K)` receives each selected key once, with
// slots 0..need-1 in unspecified order.  Requires 1 <= need <= #items.
// When `prestashed` >= 0 the caller has already put all `prestashed` items'
// keys into sm.stash (and synchronized), and `src` is never read.
//
// Rounds: histogram the next digit of the items in the current region, find
// the boundary digit, commit strictly better digits, retain the boundary
// group.  As soon as the boundary group fits STASH_CAP it is copied on chip
// (and everything above it emitted) so that later rounds never touch `src`.
template <int NT, class SM, class Src, class Emit>
__device__ void exact_select(SM &sm, Src &src, uint32_t need, Emit &&emit, int prestashed = -1)
{
    const int tid = threadIdx.x;
    if (tid == 0) {
        sm.P = 0; sm.M = 0; sm.quota = need; sm.level = 0;
        sm.done = 0; sm.out_n = 0;
        sm.stashed = prestashed >= 0 ? 1u : 0u;
        sm.stash_n = prestashed >= 0 ? (uint32_t)prestashed : 0u;
    }
    __syncthreads();
    for (;;) {
        for (int i = tid; i < NBINS; i += NT) sm.hist[i] = 0u;
        __syncthreads();
        const uint64_t P = sm.P, M = sm.M;
        const int lvl = (int)sm.level;
        if (sm.stashed) {
            const uint32_t n = sm.stash_n;
            for (uint32_t i = tid; i < n; i += NT) {
                const uint64_t K = sm.stash[i];
                if ((K & M) == P) atomicAdd(&sm.hist[key_digit(lvl, K)], 1u);
            }
        } else {
            src.for_each([&](uint32_t idx, float v) {
                const uint64_t K = make_key(v, idx);
                if ((K & M) == P) atomicAdd(&sm.hist[key_digit(lvl, K)], 1u);
            });
        }
        __syncthreads();
        find_boundary<NT>(sm.hist, sm.quota, sm.scan, &sm.b);
        if (tid == 0) {
            const uint32_t q = sm.quota - sm.b.above;
            sm.quota = q;
            sm.P = P | ((uint64_t)sm.b.digit << level_shift(lvl));
            sm.M = M | level_mask(lvl);
            sm.level = (uint32_t)(lvl + 1);
            sm.done = (sm.b.eq <= q || lvl == 5) ? 1u : 0u;
        }
        __syncthreads();
        const uint64_t P2 = sm.P, M2 = sm.M;
        if (sm.done) {
            // Everything at or above the resolved prefix is the answer.
            if (sm.stashed) {
                const uint32_t n = sm.stash_n;
                for (uint32_t i0 = 0; i0 < n; i0 += NT) {
                    const uint32_t i = i0 + tid;
                    const uint64_t K = i < n ? sm.stash[i] : 0ull;
                    const bool take = i < n && (K & M2) >= P2;
                    const uint32_t slot = wave_reserve(take, &sm.out_n);
                    if (take) emit(slot, K);
                }
            } else {
                src.for_each([&](uint32_t idx, float v) {
                    const uint64_t K = make_key(v, idx);
                    const bool take = (K & M2) >= P2;
                    const uint32_t slot = wave_reserve(take, &sm.out_n);
                    if (take) emit(slot, K);
                });
            }
            __syncthreads();
            return;
        }
        if (!sm.stashed && sm.b.eq <= (uint32_t)SM::cap) {
            src.for_each([&](uint32_t idx, float v) {
                const uint64_t K = make_key(v, idx);
                const uint64_t km = K & M2;
                const bool above = km > P2;
                const bool keep = km == P2;
                const uint32_t slot = wave_reserve(above, &sm.out_n);
                if (above) emit(slot, K);
                const uint32_t s = wave_reserve(keep, &sm.stash_n);
                if (keep && s < (uint32_t)SM::cap) sm.stash[s] = K;
            });
            __syncthreads();
            if (tid == 0) sm.stashed = 1u;
            __syncthreads();
        }
    }
}

// Item source of exact_select calls that start from a filled stash.
struct NoSrc {
    template <class F>
    __device__ void for_each(F &&) const {}
};

// Exact Top-`need` of the `n` items whose composite keys the caller has put
// into sm.stash (n <= SM::cap, 1 <= need <= n, followed by a barrier).
//
// A value histogram first narrows the problem: NBINS equal-width bins over
// the items' own [min, max] (a monotone map of the value, so the order of
// bins is the order of values), the boundary bin b where the count from the
// top reaches `need`, every item of a better bin emitted at once, and the
// items of bin b gathered.  Only those go through the composite-key radix
// rounds (value digits, then inverted-index digits), which settle the exact
// boundary including the lower-index rule for equal values.  When the range
// is degenerate or the boundary bin is too large to gather, the radix rounds
// run over all n items instead.
template <int NT, class SM, class Emit>
__device__ __forceinline__ void select_stashed(SM &sm, uint32_t n, uint32_t need, Emit &&emit, bool range_ready = false)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    NoSrc nosrc;
    // every loop below reads its LDS items in batches of SB per thread, so
    // that a thread waits for one LDS round trip per batch, not per item
    constexpr int SB = 4;
    if (!range_ready) {  // value range (else each wave's was stored while gathering)
        float mn = __builtin_inff(), mx = -__builtin_inff();
        for (uint32_t i0 = tid; i0 < n; i0 += SB * NT) {
            float v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const uint32_t i = i0 + j * NT;
                v[j] = i < n ? key_value(sm.stash[i]) : __builtin_nanf("");
            }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                mn = fminf(mn, v[j]);  // fminf/fmaxf ignore the NaN padding
                mx = fmaxf(mx, v[j]);
            }
        }
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane == 0) {
            sm.vmin[wave] = mn;
            sm.vmax[wave] = mx;
        }
    }
    for (int i = tid; i < NBINS; i += NT) sm.hist[i] = 0u;
    if (tid == 0) sm.n_bound = 0;
    __syncthreads();
    float mn = sm.vmin[0], mx = sm.vmax[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        mn = fminf(mn, sm.vmin[w]);
        mx = fmaxf(mx, sm.vmax[w]);
    }
    const float scale = (float)NBINS / (mx - mn);
    const bool binned = mx > mn && __builtin_isfinite(scale) && scale > 0.f && __builtin_isfinite(mn);
    if (!binned) {
        exact_select<NT>(sm, nosrc, need, emit, (int)n);
        return;
    }
    auto bin_of_value = [&](float v) {
        return (uint32_t)fminf(fmaxf(floorf((v - mn) * scale), 0.f), (float)(NBINS - 1));
    };
    for (uint32_t i0 = tid; i0 < n; i0 += SB * NT) {
        uint32_t b[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const uint32_t i = i0 + j * NT;
            b[j] = i < n ? bin_of_value(key_value(sm.stash[i])) : NBINS;
        }
#pragma unroll
        for (int j = 0; j < SB; ++j)
            if (b[j] < (uint32_t)NBINS) atomicAdd(&sm.hist[b[j]], 1u);
    }
    __syncthreads();
    find_boundary<NT>(sm.hist, need, sm.scan, &sm.b);
    const uint32_t B = sm.b.digit, above = sm.b.above, eq = sm.b.eq;
    if (eq > (uint32_t)BOUND_CAP) {
        exact_select<NT>(sm, nosrc, need, emit, (int)n);
        return;
    }
    if (tid == 0) sm.out_n = 0;
    __syncthreads();
    {
        // count this thread's items above / at the boundary bin, reserve the
        // slots once, then write them
        uint32_t nt = 0, nk = 0;
        for (uint32_t i0 = tid; i0 < n; i0 += SB * NT) {
            uint32_t b[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const uint32_t i = i0 + j * NT;
                b[j] = i < n ? bin_of_value(key_value(sm.stash[i])) : 0u;
                nt += i < n && b[j] > B;
                nk += i < n && b[j] == B;
            }
        }
        uint32_t st = wave_reserve_n(nt, &sm.out_n);
        uint32_t sk = wave_reserve_n(nk, &sm.n_bound);
        for (uint32_t i0 = tid; i0 < n; i0 += SB * NT) {
            uint64_t K[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const uint32_t i = i0 + j * NT;
                K[j] = i < n ? sm.stash[i] : 0ull;
            }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                if (i0 + j * NT >= n) continue;
                const uint32_t b = bin_of_value(key_value(K[j]));
                if (b > B) emit(st++, K[j]);
                else if (b == B) sm.bound[sk++] = K[j];
            }
        }
    }
    __syncthreads();
    const uint32_t q = need - above;  // 1 <= q <= eq
    if (q == eq) {
        for (uint32_t i = tid; i < eq; i += NT) emit(above + i, sm.bound[i]);
        __syncthreads();
        return;
    }
    if (eq <= (uint32_t)RANK_CAP) {
        // A small boundary bin: every item's rank among the bin's items (all
        // composite keys are distinct) decides it directly; items ranked
        // below q fill slots above + rank.
        if ((uint32_t)tid < eq) {
            const uint64_t K = sm.bound[tid];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < eq; ++j) rank += sm.bound[j] > K ? 1u : 0u;
            if (rank < q) emit(above + rank, K);
        }
        __syncthreads();
        return;
    }
    for (uint32_t i = tid; i < eq; i += NT) sm.stash[i] = sm.bound[i];
    __syncthreads();
    exact_select<NT>(sm, nosrc, q, [&](uint32_t slot, uint64_t K) { emit(above + slot, K); }, (int)eq);
}

}  // namespace itk
