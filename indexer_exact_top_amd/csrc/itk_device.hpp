// Device building blocks shared by the standalone and the fused Top-k.
//
//  * ordered fp32 keys and the 64-bit composite key (value, inverted index)
//    whose descending order is "score descending, index ascending";
//  * the 11-bit coarse key of the sampled view (Sample-Guided Exact Top-K,
//    Sec. 4.2: the fp16 ordered key shifted right by 5, 2^11 bins) and the
//    inclusive fp32 endpoint of a coarse bin (Sec. 5.2);
//  * a block-wide boundary search over a 2048-bin LDS histogram;
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

constexpr int NBINS = 2048;       // one 2^11-bin histogram, reused by every round
constexpr int STASH_CAP = 4096;   // boundary-group entries kept on chip

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

// Smallest fp32 value x (over [-inf, +inf]) with coarse_key(x) >= tau: then
// "x >= endpoint" reproduces "coarse_key(x) >= tau" with one compare.  Bins
// above the bin of +inf hold only NaN codes; their endpoint is NaN, which
// admits no value.
__device__ inline float coarse_endpoint(uint32_t tau)
{
    uint32_t lo = ordered_key(-__builtin_inff());
    uint32_t hi = ordered_key(__builtin_inff());
    if (coarse_key(from_ordered_key(lo)) >= tau) return -__builtin_inff();
    if (coarse_key(from_ordered_key(hi)) < tau) return __builtin_nanf("");
    while (hi - lo > 1u) {  // coarse(lo) < tau <= coarse(hi)
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (coarse_key(from_ordered_key(mid)) >= tau) hi = mid;
        else lo = mid;
    }
    return from_ordered_key(hi);
}

// ---------------------------------------------------------- wave helpers
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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
        base = __shfl(base, leader);
    }
    return base + lanes_below(m);
}

// Inclusive suffix sum over the lanes of a wave: lane l gets sum_{l' >= l} v.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v)
{
    const int l = (int)lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(v, off);
        if (l + off < 64) v += o;
    }
    return v;
}

// ------------------------------------------------- block boundary search
struct BoundaryOut {
    uint32_t digit;  // boundary bin
    uint32_t above;  // items in bins > digit
    uint32_t eq;     // items in the boundary bin
    uint32_t total;  // items in all bins
};

// d = max{b : sum_{b' >= b} hist[b'] >= quota}.  When quota exceeds the
// total, d = 0 and above + eq == total.  Block of NT threads; `scan` holds
// NT/64 words.  Ends with a barrier; the result is in `out` for every thread.
template <int NT>
__device__ void find_boundary(const uint32_t *hist, uint32_t quota, uint32_t *scan, BoundaryOut *out)
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
    if (tid == 0 && total < quota) {
        out->digit = 0;
        out->above = total - hist[0];
        out->eq = hist[0];
        out->total = total;
    }
    if (excl < quota && excl + s >= quota) {
        uint32_t cum = excl;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            if (cum + loc[i] >= quota) {
                out->digit = (uint32_t)(tid * PER + i);
                out->above = cum;
                out->eq = loc[i];
                out->total = total;
                break;
            }
            cum += loc[i];
        }
    }
    __syncthreads();
}

// --------------------------------------------------------- exact select
struct SelectSmem {
    uint32_t hist[NBINS];
    uint64_t stash[STASH_CAP];
    uint64_t P, M;        // resolved prefix and its mask
    uint32_t quota;       // items still to take from the current region
    uint32_t level;
    uint32_t done, stashed, stash_n, out_n;
    BoundaryOut b;
    uint32_t scan[16];
};

// Exact Top-`need` of the items produced by `src` under the composite key.
//
// `src.for_each(f)` must call f(index, value) exactly once per item, spread
// over the threads of the block (every thread must call for_each; it may
// contain barriers).  `emit(slot, K)` receives each selected key once, with
// slots 0..need-1 in unspecified order.  Requires 1 <= need <= #items.
//
// Rounds: histogram the next digit of the items in the current region, find
// the boundary digit, commit strictly better digits, retain the boundary
// group.  As soon as the boundary group fits STASH_CAP it is copied on chip
// (and everything above it emitted) so that later rounds never touch `src`.
template <int NT, class Src, class Emit>
__device__ void exact_select(SelectSmem &sm, Src &src, uint32_t need, Emit &&emit)
{
    const int tid = threadIdx.x;
    if (tid == 0) {
        sm.P = 0; sm.M = 0; sm.quota = need; sm.level = 0;
        sm.done = 0; sm.stashed = 0; sm.stash_n = 0; sm.out_n = 0;
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
        if (!sm.stashed && sm.b.eq <= (uint32_t)STASH_CAP) {
            src.for_each([&](uint32_t idx, float v) {
                const uint64_t K = make_key(v, idx);
                const uint64_t km = K & M2;
                const bool above = km > P2;
                const bool keep = km == P2;
                const uint32_t slot = wave_reserve(above, &sm.out_n);
                if (above) emit(slot, K);
                const uint32_t s = wave_reserve(keep, &sm.stash_n);
                if (keep && s < (uint32_t)STASH_CAP) sm.stash[s] = K;
            });
            __syncthreads();
            if (tid == 0) sm.stashed = 1u;
            __syncthreads();
        }
    }
}

}  // namespace itk
