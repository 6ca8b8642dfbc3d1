// Standalone exact Top-k over materialized ragged fp32 rows (gfx950).
//
// Follows the three phases of the Sample-Guided Exact Top-K paper
// (arXiv 2609.08450, Sec. 4), re-mapped onto CDNA4, with two of the
// execution mappings of its Sec. 5.5 chosen on the host by shape:
//
//  k_ragged_rowlocal  many rows (at least RAG_RL_MIN_ROWS) of at most
//                   RAG_RL_MAX_PITCH scores, and k small enough that the
//                   expected candidates fit on chip: one workgroup per row
//                   does everything in one launch.  The
//                   row's first chunks of 16-byte loads are issued, then the
//                   block-strided view (Sec. 4.2) gives the coarse boundaries
//                   and their inclusive fp32 endpoints (Sec. 5.2); the row
//                   streams through registers in double-buffered chunks, and
//                   values at or above the primary endpoint go straight into
//                   the on-chip candidate stash (per chunk: a count per lane,
//                   one LDS atomic per wave, then the writes).  The refinement
//                   (Sec. 5.4) runs on the stash; an underfilled view takes a
//                   band pass over the row, an overflowing one the exact route
//                   (Sec. 4.3, Table 2).  No global scratch, no second
//                   launch; the hardware dispatcher hands rows to CUs as they
//                   free up, which balances ragged lengths.  A row whose
//                   valid entries all fit the stash skips the view and goes
//                   whole into the stash (the direct-exact row-local mapping
//                   of Sec. 5.5): rows of a pitch that fits take this
//                   kernel at any row count, with a smaller stash for
//                   short pitches (more workgroups per CU).
//
// Longer rows (decoding against long contexts) are cut into segments:
//
//  k_ragged_scan    one workgroup per (row, segment).  Phase 1: every segment
//                   rebuilds the same block-strided view of its row (Sec. 4.2
//                   and the KV-split mapping of Sec. 5.5), histograms the
//                   11-bit coarse key in LDS, locates the primary and
//                   secondary boundaries tau0/tau1 and turns them into
//                   inclusive fp32 endpoints (Sec. 5.2).  Phase 2: one pass
//                   over the segment with 16-byte non-temporal loads (the
//                   first batch issued before phase 1, later ones double-
//                   buffered) compares each value with the primary endpoint
//                   (Sec. 5.3); admitted values are appended to a per-wave
//                   slice whose slots come from a compare mask + popcount +
//                   lane rank (no atomics).
//  k_ragged_finish  one workgroup per row.  Sums the per-wave counts and
//                   picks the route: certified primary, band pass (Sec. 4.3
//                   "Underfilled views"; the pass also counts the values
//                   between the endpoints, which gives C(tau1)), or the exact
//                   route over the whole row (Table 2).  Then the candidates
//                   are gathered on chip and refined (Sec. 5.4), and the
//                   indices written.
//
// The view samples 16 consecutive elements (one 64-byte segment) out of every
// 16*s: 1/s of the row like a single-element stride, but every sampled byte
// shares a cache line with its neighbours instead of pulling a whole line for
// one float.
#include "itk_device.hpp"
#include "itk_internal.hpp"

namespace itk {

struct RaggedArgs {
    const float *scores;
    const int32_t *row_len;
    int32_t *out_idx;
    int32_t *route;
    uint32_t *cnt;   // [M][P][W] admitted per (segment, wave); may exceed subcap
    float4 *ep;      // [M] {e0, e1, admit_all, 0}
    Cand *slices;    // [M][P][W][subcap]
    Cand *band;      // [M][bandcap]
    int64_t pitch, seg;
    int32_t M, k, P, subcap, bandcap, view_blocks, force;
    int32_t rlcap;   // row-local route: candidates kept on chip (<= STASH_CAP)
    uint32_t direct_max;  // row-local route: rows of at most this many scores are selected whole (no view)
    int32_t *order;  // row-local route: [M] rows by descending length (workgroup b takes row order[b]),
                     // or null: workgroup b takes row b
    float rho, rho1;
};

__device__ __forceinline__ uint32_t row_length(const RaggedArgs &a, int r)
{
    int32_t L = a.row_len[r];
    if (L < 0) L = 0;
    if ((int64_t)L > a.pitch) L = (int32_t)a.pitch;
    return (uint32_t)L;
}

template <bool VEC>
__global__ __launch_bounds__(RAG_THREADS) void k_ragged_scan(RaggedArgs a)
{
    __shared__ uint32_t hist[NBINS];
    __shared__ uint32_t scan_tmp[16];
    __shared__ BoundaryOut bq[2];  // primary, secondary boundary
    __shared__ float s_e[2];

    // the wave index is read into a scalar register, so that the slice
    // address and its buffer resource below are known to be wave-uniform
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const uint32_t L = row_length(a, r);
    const int64_t seg_lo = (int64_t)p * a.seg;
    const int64_t seg_hi = (seg_lo + a.seg < (int64_t)L) ? seg_lo + a.seg : (int64_t)L;
    const size_t cell = ((size_t)r * a.P + p) * RAG_WAVES + wave;

    if ((seg_lo >= (int64_t)L && p != 0) || a.force == 1) {
        if (a.force == 1 && p == 0 && tid == 0) a.ep[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane == 0) a.cnt[cell] = 0u;
        return;
    }
    const float *row = a.scores + (size_t)r * (size_t)a.pitch;

    // The segment's first batch of 16-byte loads is issued before phase 1,
    // so that its memory latency overlaps the view pass; later batches are
    // double-buffered against the classification of the previous one.
    constexpr int U = RAG_U;
    constexpr uint32_t BATCH = (uint32_t)RAG_THREADS * U;  // float4 per batch
    const uint32_t n4 = (VEC && seg_hi > seg_lo) ? (uint32_t)((seg_hi - seg_lo) >> 2) : 0u;
    const f32x4_t *v4 = reinterpret_cast<const f32x4_t *>(row + seg_lo);
    auto load_batch = [&](f32x4_t (&x)[U], uint32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = base + u * RAG_THREADS + tid;
            // NaN past the segment: it passes no comparison
            const float nan = __builtin_nanf("");
            x[u] = j < n4 ? __builtin_nontemporal_load(v4 + j) : f32x4_t{nan, nan, nan, nan};
        }
    };
    f32x4_t xa[U], xb[U];
    if (n4) load_batch(xa, 0);

    // ---- Phase 1: block-strided view -> coarse histogram -> endpoints.
    for (int i = tid; i < NBINS; i += RAG_THREADS) hist[i] = 0u;
    __syncthreads();
    const uint32_t sb = (uint32_t)a.view_blocks;
    const uint32_t phase = (uint32_t)r % sb;
    const uint32_t nb_total = (L + 15u) >> 4;
    const uint32_t nvb = nb_total > phase ? (nb_total - 1u - phase) / sb + 1u : 0u;
    for (uint32_t e0 = 0; e0 < nvb * 16u; e0 += RAG_THREADS * 8u) {
        float x[8];  // all of a thread's view loads in flight at once
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t e = e0 + j * RAG_THREADS + tid;
            const uint32_t i = (phase + (e >> 4) * sb) * 16u + (e & 15u);
            x[j] = (e < nvb * 16u && i < L) ? row[i] : __builtin_nanf("");
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (x[j] == x[j]) atomicAdd(&hist[coarse_key(x[j])], 1u);
    }
    __syncthreads();
    uint32_t n_a = 0;
    if (nvb) {
        const uint32_t last = (phase + (nvb - 1u) * sb) * 16u;
        n_a = (nvb - 1u) * 16u + ((L - last) < 16u ? (L - last) : 16u);
    }
    const double frac = L ? (double)n_a / (double)L : 0.0;
    const uint32_t q0 = (uint32_t)ceil((double)a.rho * a.k * frac);
    const uint32_t q1 = (uint32_t)ceil((double)a.rho1 * a.k * frac);
    const bool admit_all = (n_a < q1) || q0 == 0u || ((double)a.rho1 * a.k >= (double)L);
    if (!admit_all) {
        const uint32_t qs[2] = {q0, q1};
        find_boundaries<RAG_THREADS, 2>(hist, qs, scan_tmp, bq);
    }
    if (wave < 2) {  // wave 0: primary endpoint, wave 1: secondary
        const float e = admit_all ? -__builtin_inff() : coarse_endpoint_wave(bq[wave].digit);
        if (lane == 0) s_e[wave] = e;
    }
    __syncthreads();
    if (tid == 0 && p == 0) a.ep[r] = make_float4(s_e[0], s_e[1], admit_all ? 1.f : 0.f, 0.f);
    const float e0 = s_e[0];

    // ---- Phase 2: certify + collect over [seg_lo, seg_hi).
    // The wave's slice is addressed through a buffer resource whose range is
    // the slice: stores past its capacity are dropped by the hardware range
    // check.  The count keeps growing, and a count above the capacity sends
    // the row to the exact route, which ignores the slice.
    Cand *slice = a.slices + cell * (size_t)a.subcap;
    const __amdgpu_buffer_rsrc_t srd =
        __builtin_amdgcn_make_buffer_rsrc(slice, 0, (int)(a.subcap * (int)sizeof(Cand)), BUF_RSRC_WORD3);
    uint32_t cnt = 0;   // wave-uniform: admitted so far
    // One score: an admitted score takes the next slot of the wave's slice
    // (compare mask + lane rank).  Positions past the segment hold NaN, which
    // no comparison admits.  The secondary count C(tau1) is not taken here:
    // the finisher needs it only for an underfilled row, and then takes it in
    // its band pass.
    auto classify = [&](uint32_t i, float x) {
        const uint64_t m0 = __builtin_amdgcn_fcmpf(x, e0, 3);  // ordered >=, as a lane mask
        if (x >= e0) {
            const uint32_t slot =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m0, cnt));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{i, __float_as_uint(x)}, srd, slot * (uint32_t)sizeof(Cand),
                                                  0, 0);
        }
        cnt += (uint32_t)__builtin_popcountll(m0);
    };
    if (seg_hi > seg_lo) {
        if (VEC) {
            auto classify_batch = [&](const f32x4_t (&x)[U], uint32_t base) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t i0 = (uint32_t)seg_lo + 4u * (base + u * RAG_THREADS + tid);
                    classify(i0 + 0u, x[u].x);
                    classify(i0 + 1u, x[u].y);
                    classify(i0 + 2u, x[u].z);
                    classify(i0 + 3u, x[u].w);
                }
            };
            for (uint32_t base = 0; base < n4; base += 2 * BATCH) {
                if (base + BATCH < n4) load_batch(xb, base + BATCH);
                classify_batch(xa, base);
                if (base + BATCH < n4) {
                    if (base + 2 * BATCH < n4) load_batch(xa, base + 2 * BATCH);
                    classify_batch(xb, base + BATCH);
                }
            }
            const uint32_t rem_lo = (uint32_t)seg_lo + 4u * n4;
            if (wave == 0 && rem_lo < (uint32_t)seg_hi) {
                const uint32_t i = rem_lo + lane;
                classify(i, i < (uint32_t)seg_hi ? row[i] : __builtin_nanf(""));
            }
        } else {
            for (int64_t base = seg_lo; base < seg_hi; base += RAG_THREADS) {
                const int64_t i = base + tid;
                classify((uint32_t)i, i < seg_hi ? row[i] : __builtin_nanf(""));
            }
        }
    }
    if (lane == 0) a.cnt[cell] = cnt;
}

// Items of a row's candidate slices (and band slice), for exact_select.
struct SliceSrc {
    const Cand *slices;     // [ncells][subcap]
    const uint32_t *cnt;    // [ncells]
    int ncells;
    uint32_t subcap;
    const Cand *band;
    uint32_t band_n;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        for (int c = 0; c < ncells; ++c) {
            const uint32_t n = cnt[c] < subcap ? cnt[c] : subcap;
            const Cand *s = slices + (size_t)c * subcap;
            for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
                const Cand e = s[i];
                f(e.idx, e.val);
            }
        }
        for (uint32_t i = threadIdx.x; i < band_n; i += blockDim.x) {
            const Cand e = band[i];
            f(e.idx, e.val);
        }
    }
};

// Every valid entry of one row.
struct RowSrc {
    const float *row;
    uint32_t L;
    bool vec;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        if (vec) {
            const uint32_t n4 = L >> 2;
            const float4 *v4 = reinterpret_cast<const float4 *>(row);
            for (uint32_t j = threadIdx.x; j < n4; j += blockDim.x) {
                const float4 x = v4[j];
                f(4u * j + 0u, x.x);
                f(4u * j + 1u, x.y);
                f(4u * j + 2u, x.z);
                f(4u * j + 3u, x.w);
            }
            for (uint32_t i = 4u * n4 + threadIdx.x; i < L; i += blockDim.x) f(i, row[i]);
        } else {
            for (uint32_t i = threadIdx.x; i < L; i += blockDim.x) f(i, row[i]);
        }
    }
};

enum { ROUTE_SAMPLE = 1, ROUTE_BAND = 2, ROUTE_EXACT = 3, ROUTE_ALL = 4 };

// Copies every candidate of a row (slices in cell order, then the band
// slice) into the on-chip stash as composite keys; returns the count.  The
// caller guarantees that the count fits STASH_CAP and that cpre holds the
// prefix of the per-cell counts (cpre[c] <= item < cpre[c + 1] for the items
// of cell c).  With at most two cells per wave, each wave copies whole cells
// (all of a lane's loads of a cell issued before any is consumed).  With more
// cells, item i is located by a fixed-step binary search over cpre in LDS, so
// that every thread keeps B independent loads in flight whatever the cells'
// sizes (measured on one row of 2^20 scores in 64 segments: 4.2 us against
// 16 round trips for the per-wave copy; the per-wave copy is about 1 us
// faster with 8 segments).  The value range is taken on the way
// (select_stashed reads it).
__device__ uint32_t gather_candidates(const SliceSrc &src, const uint32_t *cpre, SelectSmem &sm)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = blockDim.x, nw = nt >> 6;
    const uint32_t nslice = cpre[src.ncells], total = nslice + src.band_n;
    constexpr int B = 8;  // loads in flight per thread
    float mn = __builtin_inff(), mx = -__builtin_inff();
    auto put = [&](uint32_t i, const Cand &e) {
        sm.stash[i] = make_key(e.val, e.idx);
        mn = fminf(mn, e.val);
        mx = fmaxf(mx, e.val);
    };
    if (src.ncells <= 2 * nw) {
        for (int c = wave; c < src.ncells; c += nw) {
            const uint32_t lo = cpre[c], n = cpre[c + 1] - lo;
            const Cand *cell = src.slices + (size_t)c * src.subcap;
            for (uint32_t i0 = 0; i0 < n; i0 += 64 * B) {
                Cand e[B];
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    const uint32_t i = i0 + j * 64 + lane;
                    if (i < n) e[j] = cell[i];
                }
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    const uint32_t i = i0 + j * 64 + lane;
                    if (i < n) put(lo + i, e[j]);
                }
            }
        }
    } else {
        for (uint32_t i0 = tid; i0 < nslice; i0 += B * nt) {
            Cand e[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint32_t i = i0 + j * nt;
                if (i < nslice) {
                    // largest lo < ncells with cpre[lo] <= i, in a fixed
                    // number of steps, so that the B searches interleave
                    // (every index read stays below RAG_MAX_CELLS)
                    int lo = 0;
#pragma unroll
                    for (int step = RAG_MAX_CELLS / 2; step >= 1; step >>= 1)
                        if (lo + step < src.ncells && cpre[lo + step] <= i) lo += step;
                    e[j] = src.slices[(size_t)lo * src.subcap + (i - cpre[lo])];
                }
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint32_t i = i0 + j * nt;
                if (i < nslice) put(i, e[j]);
            }
        }
    }
    for (uint32_t i0 = tid; i0 < src.band_n; i0 += B * nt) {
        Cand e[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t i = i0 + j * nt;
            if (i < src.band_n) e[j] = src.band[i];
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t i = i0 + j * nt;
            if (i < src.band_n) put(nslice + i, e[j]);
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        sm.vmin[wave] = mn;
        sm.vmax[wave] = mx;
    }
    __syncthreads();
    return total;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_ragged_finish(RaggedArgs a, int vec)
{
    static_assert(RAG_MAX_CELLS <= NT, "one cell per thread in the count prefix");
    __shared__ SelectSmem sm;
    __shared__ uint32_t s_c0, s_ovf, s_band_n;
    __shared__ uint32_t s_wsum[NT / 64];
    __shared__ uint32_t cpre[RAG_MAX_CELLS + 1];

    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int ncells = a.P * RAG_WAVES;
    const size_t cell0 = (size_t)r * ncells;
    // independent loads first: one memory round trip for all of them
    const uint32_t L = row_length(a, r);
    const float4 ep = a.ep[r];
    const bool has_cell = tid < ncells;
    const uint32_t my_cnt = has_cell ? a.cnt[cell0 + tid] : 0u;
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    int32_t *out = a.out_idx + (size_t)r * a.k;
    for (uint32_t i = need + tid; i < (uint32_t)a.k; i += NT) out[i] = -1;
    if (need == 0) {
        if (tid == 0 && a.route) a.route[r] = ROUTE_ALL;
        return;
    }
    if (tid == 0) { s_c0 = 0; s_ovf = 0; s_band_n = 0; }
    __syncthreads();
    // Total admitted count C0 and the overflow flag; with at most one cell
    // per thread, also the prefix of the stored (capped) counts, cpre.
    const bool on_chip_cells = ncells <= RAG_MAX_CELLS;
    for (int c = tid; c < ncells; c += NT) {
        const uint32_t n = c == tid ? my_cnt : a.cnt[cell0 + c];
        atomicAdd(&s_c0, n);
        if (n > (uint32_t)a.subcap) atomicOr(&s_ovf, 1u);
    }
    uint32_t incl = 0;
    if (on_chip_cells) {
        incl = wave_incl_sum(min(my_cnt, (uint32_t)a.subcap));
        if ((tid & 63) == 63) s_wsum[tid >> 6] = incl;
    }
    __syncthreads();
    if (on_chip_cells) {
        uint32_t off = 0;
        for (int w = 0; w < (tid >> 6); ++w) off += s_wsum[w];
        if (has_cell) cpre[tid + 1] = off + incl;
        if (tid == 0) cpre[0] = 0;
    }
    const float *row = a.scores + (size_t)r * (size_t)a.pitch;
    const uint32_t C0 = s_c0;
    int route = ROUTE_BAND;  // underfilled, or the sample route forced off
    if (a.force == 1 || s_ovf) route = ROUTE_EXACT;
    else if (C0 >= need && a.force != 2) route = ep.z != 0.f ? ROUTE_ALL : ROUTE_SAMPLE;

    if (route == ROUTE_BAND) {
        // Second traversal: append the values admitted by the secondary
        // endpoint but not by the primary one, and count them all, so that
        // C(tau1) = C0 + band count.  The band route holds when C(tau1)
        // reaches the quota and the band fits its slice; otherwise the row
        // takes the exact route.
        Cand *band = a.band + (size_t)r * a.bandcap;
        const float e0 = ep.x, e1 = ep.y;
        RowSrc rs{row, L, vec != 0};
        rs.for_each([&](uint32_t i, float x) {
            const bool in = x >= e1 && !(x >= e0);
            const uint32_t slot = wave_reserve(in, &s_band_n);
            if (in && slot < (uint32_t)a.bandcap) band[slot] = Cand{i, x};
        });
        __syncthreads();
        if (C0 + s_band_n < need || s_band_n > (uint32_t)a.bandcap) route = ROUTE_EXACT;
    }

    auto emit = [&](uint32_t slot, uint64_t K) {
        if (slot < need) out[slot] = (int32_t)key_index(K);
    };
    if (route == ROUTE_EXACT) {
        RowSrc src{row, L, vec != 0};
        exact_select<NT>(sm, src, need, emit);
    } else {
        SliceSrc src{a.slices + cell0 * (size_t)a.subcap, a.cnt + cell0, ncells, (uint32_t)a.subcap,
                     a.band + (size_t)r * a.bandcap, route == ROUTE_BAND ? min(s_band_n, (uint32_t)a.bandcap) : 0u};
        // the slices and the band slice hold at most this many entries
        const uint32_t bound = route == ROUTE_BAND ? C0 + s_band_n : C0;
        if (bound <= (uint32_t)STASH_CAP && on_chip_cells) {
            __syncthreads();  // cpre complete
            const uint32_t n = gather_candidates(src, cpre, sm);
            select_stashed<NT>(sm, n, need, emit, true);
        } else {
            exact_select<NT>(sm, src, need, emit);
        }
    }
    if (tid == 0 && a.route) a.route[r] = route;
}


// ------------------------------------------------------------ row-local
// One workgroup of RL_THREADS per row (see the header).  Chunks of RL_U
// 16-byte loads per thread are double-buffered in registers.
// Longest rows first: workgroup b of the row-local pass takes row order[b],
// the rows sorted by descending length (counting sort over RL_ORDER_BINS
// length buckets; rows within a bucket in any order).  The dispatcher starts
// workgroups in index order and hands the next one to whichever CU frees up,
// so the long rows start first and the short ones fill the tail (longest
// processing time first).  In index order, 1024 rows of 8K-128K scores on
// 512 resident workgroups finish about 1.6 times later than the balanced
// schedule; longest first, within a few percent of it.
constexpr int RL_ORDER_THREADS = 1024;
constexpr int RL_ORDER_BINS = 1024;
__global__ __launch_bounds__(RL_ORDER_THREADS) void k_ragged_order(RaggedArgs a)
{
    __shared__ uint32_t cnt[RL_ORDER_BINS];
    __shared__ uint32_t s_wsum[RL_ORDER_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t span = (uint64_t)a.pitch + 1u;
    auto bin_of_row = [&](int r) {
        const uint64_t L = row_length(a, r);
        return (uint32_t)(((uint64_t)a.pitch - L) * RL_ORDER_BINS / span);  // 0 = longest
    };
    for (int i = tid; i < RL_ORDER_BINS; i += RL_ORDER_THREADS) cnt[i] = 0u;
    __syncthreads();
    for (int r = tid; r < a.M; r += RL_ORDER_THREADS) atomicAdd(&cnt[bin_of_row(r)], 1u);
    __syncthreads();
    // exclusive prefix over the bins (one bin per thread)
    static_assert(RL_ORDER_BINS == RL_ORDER_THREADS, "one bin per thread");
    const uint32_t v = cnt[tid];
    const uint32_t incl = wave_incl_sum(v);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    cnt[tid] = off + incl - v;
    __syncthreads();
    for (int r = tid; r < a.M; r += RL_ORDER_THREADS) a.order[atomicAdd(&cnt[bin_of_row(r)], 1u)] = r;
}

// CAP: on-chip stash entries (a.rlcap <= CAP).  Short pitches take a smaller
// stash, so that more workgroups share a CU: 78 KB of LDS at STASH_CAP (two
// per CU), about 49 KB at 4096 entries (three), about 33 KB at 2048 (four).
template <bool VEC, int CAP>
__global__ __launch_bounds__(RL_THREADS, 4) void k_ragged_rowlocal(RaggedArgs a)
{
    __shared__ SelectSmemT<CAP> sm;
    __shared__ BoundaryOut bq[2];  // primary, secondary boundary
    __shared__ float s_e[2];
    __shared__ uint32_t s_cnt;
    constexpr int NT = RL_THREADS;
    constexpr int U = RL_U;
    constexpr uint32_t CHUNK = (uint32_t)NT * U * 4;  // scores per chunk
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = a.order ? a.order[blockIdx.x] : (int)blockIdx.x;
    const uint32_t L = row_length(a, r);
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    int32_t *out = a.out_idx + (size_t)r * a.k;
    for (uint32_t i = need + tid; i < (uint32_t)a.k; i += NT) out[i] = -1;
    if (need == 0) {
        if (tid == 0 && a.route) a.route[r] = ROUTE_ALL;
        return;
    }
    const float *row = a.scores + (size_t)r * (size_t)a.pitch;
    const uint32_t cap = (uint32_t)a.rlcap;  // <= CAP

    // Chunk c: lane-interleaved 16-byte pieces of the row's whole pieces
    // (the last 1-3 scores of a row whose length is not a multiple of 4 are
    // admitted on their own after the chunks).  Every lane issues its U loads
    // whatever the chunk (pieces past the row re-read piece 0, which stays in
    // cache; admit_chunk ignores them by index), so that the number of loads
    // in flight is the same on every path and a chunk's data is waited for
    // with vmcnt(U) while the next chunk's loads stay in flight.  Needs
    // n4 > 0.  Without 16-byte alignment the same positions are read one
    // float at a time.
    const uint32_t n4 = L >> 2;  // whole 16-byte pieces
    auto load_chunk = [&](uint32_t c, f32x4_t (&x)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i4 = c * (CHUNK / 4) + (uint32_t)(u * NT + tid);
            const uint32_t j4 = i4 < n4 ? i4 : 0u;
            if (VEC) {
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(row) + j4);
            } else {
                const float *q = row + 4u * j4;
                x[u] = f32x4_t{q[0], q[1], q[2], q[3]};
            }
        }
    };
    f32x4_t xa[U], xb[U];
    const bool exact_only = a.force == 1;
    // Direct-exact (SGTK Sec. 5.5, the row-local exact mapping): a row whose
    // valid entries all fit the stash needs no view; every entry is admitted
    // and the refinement runs on the whole row.  One read of the row.
    const bool direct = L <= a.direct_max;
    if (!exact_only && n4) load_chunk(0, xa);

    // ---- view -> coarse histogram -> endpoints (as in the segmented scan)
    float e0 = __builtin_nanf(""), e1 = __builtin_nanf("");
    bool admit_all = false;
    if (!exact_only && direct) {
        e0 = -__builtin_inff();
        admit_all = true;
        if (tid == 0) s_cnt = 0u;
        __syncthreads();
    } else if (!exact_only) {
        for (int i = tid; i < NBINS; i += NT) sm.hist[i] = 0u;
        if (tid == 0) s_cnt = 0u;
        __syncthreads();
        const uint32_t sb = (uint32_t)a.view_blocks;
        const uint32_t phase = (uint32_t)r % sb;
        const uint32_t nb_total = (L + 15u) >> 4;
        const uint32_t nvb = nb_total > phase ? (nb_total - 1u - phase) / sb + 1u : 0u;
        for (uint32_t v0 = 0; v0 < nvb * 16u; v0 += NT * 4u) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t e = v0 + j * NT + tid;
                const uint32_t i = (phase + (e >> 4) * sb) * 16u + (e & 15u);
                x[j] = (e < nvb * 16u && i < L) ? row[i] : __builtin_nanf("");
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (x[j] == x[j]) atomicAdd(&sm.hist[coarse_key(x[j])], 1u);
        }
        __syncthreads();
        uint32_t n_a = 0;
        if (nvb) {
            const uint32_t last = (phase + (nvb - 1u) * sb) * 16u;
            n_a = (nvb - 1u) * 16u + ((L - last) < 16u ? (L - last) : 16u);
        }
        const double frac = (double)n_a / (double)L;
        const uint32_t q0 = (uint32_t)ceil((double)a.rho * a.k * frac);
        const uint32_t q1 = (uint32_t)ceil((double)a.rho1 * a.k * frac);
        admit_all = (n_a < q1) || q0 == 0u || ((double)a.rho1 * a.k >= (double)L);
        if (!admit_all) {
            const uint32_t qs[2] = {q0, q1};
            find_boundaries<NT, 2>(sm.hist, qs, sm.scan, bq);
        }
        if (wave < 2) {  // wave 0: primary endpoint, wave 1: secondary
            const float e = admit_all ? -__builtin_inff() : coarse_endpoint_wave(bq[wave].digit);
            if (lane == 0) s_e[wave] = e;
        }
        __syncthreads();
        e0 = s_e[0];
        e1 = s_e[1];
    }

    // Appends the chunk's values in [lo_edge, hi_edge) (hi_edge NaN: no upper
    // edge) to the stash: a count per lane, one LDS atomic per wave, then the
    // writes (slots at or past cap are dropped; the count keeps growing).
    float mn = __builtin_inff(), mx = -__builtin_inff();
    auto admit_chunk = [&](uint32_t c, const f32x4_t (&x)[U], float lo_edge, float hi_edge) __attribute__((always_inline)) {
        auto in = [&](float v) __attribute__((always_inline)) { return v >= lo_edge && !(v >= hi_edge); };
        uint32_t n = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = c * (CHUNK / 4) + (uint32_t)(u * NT + tid) < n4;
            if (valid)
                n += (uint32_t)in(x[u].x) + (uint32_t)in(x[u].y) + (uint32_t)in(x[u].z) + (uint32_t)in(x[u].w);
        }
        const uint32_t incl = wave_incl_sum(n);
        const uint32_t total = lane_value(incl, 63);
        if (total == 0u) return;  // wave-uniform
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&s_cnt, total);
        uint32_t slot = lane_value(base, 0) + incl - n;
        if (n == 0u) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = 4u * (c * (CHUNK / 4) + (uint32_t)(u * NT + tid));
            if (i0 >= 4u * n4) continue;  // past the row's whole pieces
            const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (in(v[q])) {
                    if (slot < cap) sm.stash[slot] = make_key(v[q], i0 + (uint32_t)q);
                    mn = fminf(mn, v[q]);
                    mx = fmaxf(mx, v[q]);
                    ++slot;
                }
            }
        }
    };
    // The row's last L % 4 scores (wave 0).
    auto admit_rest = [&](float lo_edge, float hi_edge) __attribute__((always_inline)) {
        const uint32_t i = 4u * n4 + (uint32_t)lane;
        if (wave == 0 && 4u * n4 < L) {
            const float v = i < L ? row[i] : __builtin_nanf("");
            const bool ok = v >= lo_edge && !(v >= hi_edge);
            const uint64_t m = __ballot(ok);
            if (m) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_cnt, (uint32_t)__popcll(m));
                const uint32_t slot = lane_value(base, 0) + lanes_below(m);
                if (ok) {
                    if (slot < cap) sm.stash[slot] = make_key(v, i);
                    mn = fminf(mn, v);
                    mx = fmaxf(mx, v);
                }
            }
        }
    };
    // Streams the whole row through registers (chunk 0 already in xa when
    // `first_loaded`), admitting [lo_edge, hi_edge) of every chunk.
    const uint32_t nchunks4 = (n4 + CHUNK / 4 - 1) / (CHUNK / 4);
    auto stream = [&](float lo_edge, float hi_edge, bool first_loaded) __attribute__((always_inline)) {
        if (n4) {
            if (!first_loaded) load_chunk(0, xa);
            for (uint32_t c = 0; c < nchunks4; c += 2) {
                load_chunk(c + 1, xb);  // past the row: discarded re-reads
                admit_chunk(c, xa, lo_edge, hi_edge);
                load_chunk(c + 2, xa);
                if (c + 1 < nchunks4) admit_chunk(c + 1, xb, lo_edge, hi_edge);
            }
        }
        admit_rest(lo_edge, hi_edge);
    };

    int route = ROUTE_EXACT;
    uint32_t n = 0;
    if (!exact_only) {
        stream(e0, __builtin_nanf(""), true);
        __syncthreads();
        const uint32_t C0 = s_cnt;
        if (C0 <= cap && C0 >= need && (a.force != 2 || direct)) {
            route = admit_all ? ROUTE_ALL : ROUTE_SAMPLE;
            n = C0;
        } else if (C0 <= cap) {
            // Underfilled view: a second pass appends the values between the
            // endpoints; the band route holds when C(tau1) reaches the quota
            // and fits the stash.
            stream(e1, e0, false);
            __syncthreads();
            const uint32_t C1 = s_cnt;
            if (C1 >= need && C1 <= cap) {
                route = ROUTE_BAND;
                n = C1;
            }
        }
    }
    auto emit = [&](uint32_t slot, uint64_t K) {
        if (slot < need) out[slot] = (int32_t)key_index(K);
    };
    if (route == ROUTE_EXACT) {
        __syncthreads();
        RowSrc src{row, L, VEC};
        exact_select<NT>(sm, src, need, emit);
    } else {
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane == 0) {
            sm.vmin[wave] = mn;
            sm.vmax[wave] = mx;
        }
        __syncthreads();
        select_stashed<NT>(sm, n, need, emit, true);
    }
    if (tid == 0 && a.route) a.route[r] = route;
}

static int ceil_div_i(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

RaggedPlan plan_ragged(int32_t M, int64_t pitch, int32_t k)
{
    const Knobs &kn = knobs();
    RaggedPlan p;
    p.M = M; p.pitch = pitch; p.k = k;
    int s = pitch >= 262144 ? 128 : 64;
    if (kn.sample_stride > 0) s = kn.sample_stride;
    p.view_blocks = s;
    // Primary and secondary rank multiples: 1.5 and 1.75 as long as the
    // view's sample rank q0 = rho*k/s is at least 32; below that the
    // rank estimate is too coarse (on exchangeable rows the count admitted
    // by the q-th view value is about Gamma(q, 1) * L / n_a, so q = 24 at
    // s = 128, k = 2048 underfills about 4% of rows), and rho is raised to
    // 32*s/k (rho1 = 7/6 rho), which keeps the underfill rate near 3e-4.
    const float rho_floor = 32.f * (float)s / (float)(k > 0 ? k : 1);
    const float rho_auto = rho_floor > 1.5f ? rho_floor : 1.5f;
    p.rho = kn.rho > 0.f ? kn.rho : rho_auto;
    p.rho1 = kn.rho1 > 0.f ? kn.rho1 : rho_auto * (7.f / 6.f);
    if (p.rho1 < p.rho) p.rho1 = p.rho;
    p.force = kn.force_route;
    p.bandcap = 2 * k > 2048 ? 2 * k : 2048;
    // Row-local route: enough rows to occupy the chip, rows short enough for
    // one workgroup, and a secondary count that leaves room in the on-chip
    // stash.  Tests pick a mapping with the ragged_route knob (a segment
    // count also selects the segmented route).
    // Short pitches use a smaller stash (more workgroups per CU).
    const int stash = pitch <= RL_TINY_CAP ? RL_TINY_CAP : pitch <= RL_SMALL_CAP ? RL_SMALL_CAP : STASH_CAP;
    const int rlcap = kn.capacity > 0 && kn.capacity < stash ? kn.capacity : stash;
    // A pitch that fits the stash takes the row-local mapping at any row
    // count: one launch instead of two (rows of 1K-7.7K scores, 1 to 256
    // rows: 7-12 us against 13-17 us segmented).
    const bool fits_chip = pitch <= rlcap;
    const bool rl_fits = pitch <= RAG_RL_MAX_PITCH && ((double)p.rho1 * k <= (double)RAG_RL_MAX_CAND || fits_chip);
    if (rl_fits && (kn.route_select == 2 || kn.route_select == 3 ||
                    (kn.route_select == 0 && kn.splits == 0 && (M >= RAG_RL_MIN_ROWS || fits_chip)))) {
        p.rowlocal = true;
        p.rlstash = stash;
        p.rlcap = rlcap;
        // Direct-exact rows: a row no longer than the sampled steps' expected
        // candidate count plus RAG_DIRECT_MARGIN is refined whole (the view's
        // latency exceeds refining the extra entries); route 3 takes every
        // row that fits, route 2 none.
        const double dmax = ceil((double)p.rho1 * k) + RAG_DIRECT_MARGIN;
        p.direct_max = kn.route_select == 2 ? 0u
                     : kn.route_select == 3 ? (uint32_t)rlcap
                     : (uint32_t)(dmax < (double)rlcap ? dmax : (double)rlcap);
        p.P = 1;
        p.seg = pitch;
        p.off_order = 0;
        p.bytes = align256((size_t)M * sizeof(int32_t));  // the row order; candidates stay on chip
        return p;
    }
    // Segmented route: about 512 workgroups (up to RAG_MAX_SPLITS segments
    // per row, so that a few long rows, as in decoding, still spread over the
    // chip), and below 1024 rows segments of at most 32768 scores (128 KB),
    // so that long rows do not serialize on one workgroup
    int target = ceil_div_i(512, M);
    const int by_len = ceil_div_i(pitch > 0 ? pitch : 1, RAG_SEG_MAX);
    // From 1024 rows on, one workgroup per row already fills the chip, and
    // every extra segment repeats the row's view pass (measured on 1024 rows
    // of 8K-128K scores: one segment per row 107 us, four 118 us).
    if (M < 1024 && target < by_len) target = by_len;
    if (target < 1) target = 1;
    if (target > RAG_MAX_SPLITS) target = RAG_MAX_SPLITS;
    if (kn.splits > 0) target = kn.splits;
    int64_t seg = (pitch + target - 1) / target;
    seg = ((seg + 1023) / 1024) * 1024;
    if (seg < 4096) seg = 4096;
    p.seg = seg;
    p.P = ceil_div_i(pitch > 0 ? pitch : 1, seg);
    // Each segment can hold twice the row's expected secondary count (any
    // one segment may hold all of a row's top values); past 16 segments per
    // row the per-segment share shrinks in proportion, which bounds the
    // workspace at 32 times the row's expected count.
    double segcap_d = 2.0 * p.rho1 * k;
    if (p.P > 16) segcap_d *= 16.0 / p.P;
    int segcap = (int)(segcap_d + 0.5);
    if (segcap < 2048) segcap = 2048;
    if (kn.capacity > 0) segcap = kn.capacity;
    p.subcap = (segcap + RAG_WAVES - 1) / RAG_WAVES;
    p.subcap = (p.subcap + 63) & ~63;
    const size_t cells = (size_t)M * p.P * RAG_WAVES;
    size_t off = 0;
    p.off_cnt = off; off = align256(off + cells * 4);
    p.off_ep = off; off = align256(off + (size_t)M * 16);
    p.off_slices = off; off = align256(off + cells * (size_t)p.subcap * sizeof(Cand));
    p.off_band = off; off = align256(off + (size_t)M * p.bandcap * sizeof(Cand));
    p.bytes = off;
    return p;
}

hipError_t launch_ragged(const RaggedPlan &p, const float *scores, const int32_t *row_len, int32_t *out_idx,
                         void *ws, hipStream_t stream)
{
    char *w = static_cast<char *>(ws);
    RaggedArgs a;
    a.scores = scores;
    a.row_len = row_len;
    a.out_idx = out_idx;
    const RouteSink &rs = route_sink();
    a.route = (rs.ptr && rs.rows >= p.M) ? rs.ptr : nullptr;
    a.cnt = reinterpret_cast<uint32_t *>(w + p.off_cnt);
    a.ep = reinterpret_cast<float4 *>(w + p.off_ep);
    a.slices = reinterpret_cast<Cand *>(w + p.off_slices);
    a.band = reinterpret_cast<Cand *>(w + p.off_band);
    a.pitch = p.pitch;
    a.seg = p.seg;
    a.M = p.M; a.k = p.k; a.P = p.P; a.subcap = p.subcap; a.bandcap = p.bandcap;
    a.view_blocks = p.view_blocks; a.force = p.force;
    a.rlcap = p.rlcap;
    a.direct_max = p.direct_max;
    a.order = nullptr;
    a.rho = p.rho; a.rho1 = p.rho1;
    const bool vec = (p.pitch % 4 == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15u) == 0);
    hipError_t e;
    if (p.rowlocal) {
        StageTimer st(ST_RAG_ROWLOCAL, stream);
        // Below RAG_RL_MIN_ROWS rows every workgroup is resident at once, so
        // the order would change nothing: workgroup b takes row b.  Nor is it
        // launched when every row takes the direct steps: their times vary
        // far less than those of sampled rows, and the order launch costs
        // more than it saves (8192 rows of at most 2048 scores: 58 us
        // without it, 67 us with it).
        if (p.M >= RAG_RL_MIN_ROWS && p.pitch > (int64_t)p.direct_max) {
            a.order = reinterpret_cast<int32_t *>(w + p.off_order);
            e = launch_kernel(k_ragged_order, dim3(1), dim3(RL_ORDER_THREADS), stream, a);
            if (e != hipSuccess) return e;
        }
        if (p.rlstash == RL_TINY_CAP)
            return vec ? launch_kernel(k_ragged_rowlocal<true, RL_TINY_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a)
                       : launch_kernel(k_ragged_rowlocal<false, RL_TINY_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a);
        if (p.rlstash == RL_SMALL_CAP)
            return vec ? launch_kernel(k_ragged_rowlocal<true, RL_SMALL_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a)
                       : launch_kernel(k_ragged_rowlocal<false, RL_SMALL_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a);
        return vec ? launch_kernel(k_ragged_rowlocal<true, STASH_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a)
                   : launch_kernel(k_ragged_rowlocal<false, STASH_CAP>, dim3(p.M), dim3(RL_THREADS), stream, a);
    }
    {
        StageTimer st(ST_RAG_SCAN, stream);
        e = vec ? launch_kernel(k_ragged_scan<true>, dim3(p.M * p.P), dim3(RAG_THREADS), stream, a)
                : launch_kernel(k_ragged_scan<false>, dim3(p.M * p.P), dim3(RAG_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_RAG_FINISH, stream);
        if (p.M >= FIN_MANY_ROWS)
            e = launch_kernel(k_ragged_finish<FIN_THREADS_MANY>, dim3(p.M), dim3(FIN_THREADS_MANY), stream, a,
                              vec ? 1 : 0);
        else
            e = launch_kernel(k_ragged_finish<FIN_THREADS>, dim3(p.M), dim3(FIN_THREADS), stream, a, vec ? 1 : 0);
    }
    return e;
}

}  // namespace itk
