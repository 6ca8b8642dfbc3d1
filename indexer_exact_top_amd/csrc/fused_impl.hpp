// Fused lightning-indexer score + exact Top-k (gfx950), templated on the
// operand formats and the shape class.
//
// Score (LiteTopK, arXiv 2607.11976, Sec. 2.1 Eq. (1)):
//     s[t,j] = sum_h w[t,h] * ReLU(q[t,h,:] . k[j,:])
// computed without materializing the score matrix, then selected exactly.
//
// Mapping onto CDNA4 (one wavefront owns one query, FUSED_WAVES queries per
// workgroup share every staged key tile):
//  * contraction: v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2f32 for
//    fp32 inputs; v_mfma_scale_f32_32x32x64_f8f6f4 when FP8 keys are scored
//    with per-row quantized FP8 queries).  MFMA rows are the query's heads
//    (one or two 32-head blocks), columns are 32 keys; the query's Q
//    fragments stay in VGPRs for the whole scan.  Key stages are copied once
//    per workgroup into padded, double-buffered LDS rows: 16- and 32-bit keys
//    (and FP8 keys scored as FP8) by direct global -> LDS loads, 128 keys per
//    stage for rows of up to 256 bytes; FP8 keys scored in bf16/fp16 go
//    through registers, 64 keys per stage, and are widened exactly on the
//    way.  The per-key FP8 scale is applied after the head reduction, which
//    is exact for non-negative scales.
//  * epilogue in registers: each lane owns 16 head rows of one key column per
//    32x32 block; w * max(acc, 0) is accumulated in-lane and the two half-waves
//    are combined with one cross-lane exchange, leaving lane l with the score
//    of key tile_start + l.  The MFMAs of each 32-key block are interleaved
//    with the epilogue of the block before it.
//  * sample -> filter -> refresh -> select (LiteTopK Sec. 3.2): a tile-strided
//    view of each row (or, with a history sample, a caller-given key list) is
//    scored first in two light passes: the score range, with the scores
//    stored when they fit the candidate buffer's bytes, then an equal-width
//    histogram of m = 2048 bins over [s_min, s_max].  The threshold bin
//    starts at the bin of the sample's rank-q score, q sized for rho * k of
//    the row (the rank calibration of the Sample-Guided paper, Sec. 4.2).  In
//    the scan, bin = floor((s - s_min) * delta) is one FMA; a key passes if
//    its bin is not below the threshold bin; passing keys are compacted with
//    a wave ballot + popcount + lane rank into a per-wave LDS staging list
//    that is flushed 64 entries at a time with one atomic on the row's
//    candidate tail, and counted in the wave's LDS histogram; the threshold
//    bin then moves up one bin at a time while the admitted keys strictly
//    above it number at least k.  Under key splits a split that raises its
//    bin publishes it to the row's word (atomic max) and the row's other
//    splits move up to it.
//  * recovery: rows whose candidates overflowed the buffer or fell short of
//    min(k, L) are re-scored by the whole grid (a full-row histogram on the
//    sampled bin map, then a pass that collects every key at or above its
//    k-th bin), so sampling never decides the result.
//  * select: one workgroup per row gathers the row's candidates into LDS,
//    commits every value-histogram bin above the boundary bin and settles the
//    boundary bin exactly (ranking or composite-key radix refinement); a row
//    whose boundary bin alone still overflows the buffer is re-scored there.
#pragma once

#include "itk_device.hpp"
#include "itk_internal.hpp"

namespace itk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

enum MType { M_BF16 = 0, M_F16 = 1, M_F32 = 2, M_FP8 = 3 };

template <int MT>
struct MTraits;
template <>
struct MTraits<M_BF16> {
    using frag = u32x4_t;
    static constexpr int ebytes = 2, kstep = 16, pad = 16;
};
template <>
struct MTraits<M_F16> {
    using frag = u32x4_t;
    static constexpr int ebytes = 2, kstep = 16, pad = 16;
};
template <>
struct MTraits<M_F32> {
    using frag = float;
    static constexpr int ebytes = 4, kstep = 2, pad = 16;
};
template <>
struct MTraits<M_FP8> {  // e4m3fn x e4m3fn, 64-element k-steps, 32 bytes per lane
    using frag = u32x8_t;
    static constexpr int ebytes = 1, kstep = 64, pad = 16;
};

template <int MT>
__device__ __forceinline__ f32x16_t mfma32(typename MTraits<MT>::frag a, typename MTraits<MT>::frag b, f32x16_t c)
{
    if constexpr (MT == M_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else if constexpr (MT == M_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else if constexpr (MT == M_FP8)  // both operands e4m3fn (format 0), unit block scales (E8M0 127)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8_t, a),
                                                               __builtin_bit_cast(i32x8_t, b), c, 0, 0, 0, 127, 0, 127);
    else
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Four e4m3fn codes (the bytes of `word`, lowest first) -> four bf16 or fp16
// values, two per dword, lowest first.  Uses the gfx950 scaled conversion
// with a unit scale; both 16-bit formats hold every e4m3fn value exactly.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int MT>
__device__ __forceinline__ u32x2_t fp8x4_widen(uint32_t word)
{
    if constexpr (MT == M_BF16)
        return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true))};
    else
        return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true))};
}

// Kernel configuration: Q dtype, K dtype, head blocks, head dim, ReLU.
//
// LDS key layout: one staged key row holds ROWB = D * (MFMA operand bytes)
// bytes in CH 16-byte chunks followed by one 16-byte pad slot (row stride
// ROWP = ROWB + 16).  The odd number of 16-byte slots per row rotates the
// LDS banks from row to row, so the 16-byte B-fragment reads of consecutive
// key rows fall on distinct banks while every read address stays a per-lane
// base plus a compile-time offset.
//
// Staging: 16- and 32-bit keys are copied global -> LDS by the direct
// LDS-load path (no registers, no LDS write instructions), in stages of
// STAGE_KEYS keys; FP8 keys go through registers to be widened once per
// workgroup, in stages of 64 keys, unless the queries are quantized to FP8
// too (Q8): then the raw key bytes are copied like 16-bit keys and the
// contraction runs on the FP8 matrix cores.
template <int QT_, int KT_, int HB_, int D_, bool RELU_, bool Q8_ = false>
struct FCfg {
    static constexpr int QT = QT_, KT = KT_, HB = HB_, D = D_;
    static constexpr bool RELU = RELU_, Q8 = Q8_;
    static_assert(!Q8 || KT == ITK_FP8_E4M3, "FP8 scoring needs FP8 keys");
    static constexpr int MT = Q8 ? M_FP8 : (QT == ITK_F32) ? M_F32 : (QT == ITK_BF16 ? M_BF16 : M_F16);
    using TR = MTraits<MT>;
    using frag = typename TR::frag;
    static constexpr int KS = D / TR::kstep;                 // MFMA k-steps
    static constexpr int ROWB = D * TR::ebytes;              // data bytes per staged key
    static constexpr int CH = ROWB / 16;                     // 16-byte chunks per key row
    static constexpr int SPR = CH + 1;                       // 16-byte slots per row (with pad)
    static constexpr int ROWP = SPR * 16;                    // LDS row stride
    static constexpr int kbytes = (KT == ITK_F32) ? 4 : (KT == ITK_FP8_E4M3 ? 1 : 2);
    static constexpr int qbytes = (QT == ITK_F32) ? 4 : 2;
    static constexpr bool SCALE = (KT == ITK_FP8_E4M3);
    static constexpr bool DMA = !SCALE || Q8;
    static constexpr int STAGE_KEYS = DMA ? (ROWB <= 256 ? 128 : 64) : TILE_KEYS;
    static constexpr int NSUB = STAGE_KEYS / TILE_KEYS;      // 64-key tiles per stage
    static constexpr int TILE_LDS = TILE_KEYS * ROWP;        // LDS bytes of one 64-key tile
    static constexpr int STAGE_BYTES = STAGE_KEYS * ROWP;
    static constexpr int EPT = TILE_KEYS * D / FUSED_THREADS; // FP8 staging: elements per thread
};

struct FusedArgs {
    const void *Q;
    const void *K;
    const float *k_scale;
    const float *W;
    const int32_t *kv_len;
    int32_t *out_idx;
    float *out_score;
    int32_t *route;
    int32_t *count;    // [T] candidates the selection started from (test knob), or null
    float4 *param;     // [T] {off, delta, degenerate, 0}
    float2 *mm;        // [T][Ps] {min, max} of the sampled scores
    uint32_t *hist;    // [T][NBINS] sample histogram
    uint32_t *tail;    // [T] candidates appended (may exceed cap)
    Cand *cand;        // [T][cap] (head rows) or [T][P][capS] (single head)
    float *samp;       // [T][samp_cap] scores of the sampled view (both paths)
    uint32_t *hist_r;  // [T][NBINS] full-row histogram of rows under recovery (head rows)
    uint32_t *rflag;   // [T] 1 when the row takes a recovery route (head rows: the grid-wide
                       // recovery; single head: the re-scoring kernel)
    uint32_t *gpub;    // [T] gate bin published across the key splits of a row (head rows)
    // single-head (query-column) path
    float *gate;       // [T] admission gate (score space)
    uint32_t *qcnt;    // [T][P] candidates per (query, key split); may exceed capS
    // history sample (head rows): the caller's prior key list, gathered
    const int32_t *prior;  // [n_prior] caller's key indices, or null
    int32_t *pidx;         // [np] gathered key index per entry, INT32_MAX where unusable; null = strided view
    void *Kp;              // [np] key rows of the entries (zero rows where unusable)
    float *kp_scale;       // [np] their FP8 scales (FP8 keys)
    uint32_t *pcount;      // [T] entries below the query's length
    int64_t np;            // entries, padded to whole tiles
    int32_t n_prior, rowb; // listed entries; bytes per key row
    int64_t N, span, span_s, samp_cap;
    int32_t T, H, k, cap, capS, G, P, Ps, sample_tiles, force;
    float rho;
};

__device__ __forceinline__ uint32_t kv_length(const FusedArgs &a, int t)
{
    int64_t L = a.kv_len[t];
    if (L < 0) L = 0;
    if (L > a.N) L = a.N;
    return (uint32_t)L;
}

__device__ __forceinline__ void map_group_split(int b, int G, int P, int &g, int &p)
{
    if (P % 8 == 0) {  // XCD-aware: the workgroups of one key split share an XCD (and its L2)
        const int xcd = b & 7, local = b >> 3;
        p = (local / G) * 8 + xcd;
        g = local % G;
    } else {
        g = b / P;
        p = b % P;
    }
}

// Number of sampled keys below L and the sample rank for the row.
//
// Strided view: the gate bin is the one holding the view's rank-q0 score,
// q0 = ceil(rho k n_a / L), which aims at about rho k admitted keys.
// History sample (LiteTopK Sec. 3.2 "Sampling"): the sample is a set of the
// row's own keys, so its k-th largest score cannot exceed the row's k-th
// largest, and the gate bin is the one holding that k-th sample score (q0 =
// k): every key of the row's Top-k passes it.  A row with fewer than k usable
// entries (or a degenerate sampled range) gets no gate.
struct RowSample {
    uint32_t n_a;
    bool admit_all;
    uint32_t q0;
};
__device__ __forceinline__ RowSample row_sample(const FusedArgs &a, int t, int g, uint32_t L, bool degenerate)
{
    RowSample rs;
    if (a.pidx) {
        rs.n_a = a.pcount[t];
        rs.q0 = (uint32_t)a.k;
        rs.admit_all = degenerate || rs.n_a < (uint32_t)a.k;
        return rs;
    }
    const uint32_t st = (uint32_t)a.sample_tiles, phase = (uint32_t)g % st;
    const uint32_t nt = (L + TILE_KEYS - 1) / TILE_KEYS;
    const uint32_t ns = nt > phase ? (nt - 1u - phase) / st + 1u : 0u;
    rs.n_a = 0;
    if (ns) {
        const uint32_t last = (phase + (ns - 1u) * st) * TILE_KEYS;
        rs.n_a = (ns - 1u) * TILE_KEYS + ((L - last) < (uint32_t)TILE_KEYS ? (L - last) : (uint32_t)TILE_KEYS);
    }
    const double target = (double)a.rho * (double)a.k;
    rs.q0 = L ? (uint32_t)ceil(target * (double)rs.n_a / (double)L) : 0u;
    rs.admit_all = degenerate || target >= (double)L || rs.n_a == 0u || rs.q0 == 0u || rs.q0 > rs.n_a;
    return rs;
}

// ----------------------------------------------------------- fragments
template <class C>
struct QFrags {
    typename C::frag q[C::HB][C::KS];
    float w[C::HB][16];

    __device__ void load(const FusedArgs &a, int t)
    {
        if constexpr (C::MT == M_FP8)
            load_q8(a, t);
        else
            load_16_32(a, t);
    }

    __device__ void load_16_32(const FusedArgs &a, int t)
    {
        const int l = (int)lane_id();
        const int H = a.H;
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) {
            const int head = hb * 32 + (l & 31);
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                if constexpr (C::MT == M_F32) {
                    const int d = kk * 2 + (l >> 5);
                    q[hb][kk] = head < H ? static_cast<const float *>(a.Q)[((size_t)t * H + head) * C::D + d] : 0.f;
                } else {
                    const int d0 = kk * 16 + 8 * (l >> 5);
                    const char *ptr = static_cast<const char *>(a.Q) + (((size_t)t * H + head) * C::D + d0) * 2;
                    q[hb][kk] = head < H ? *reinterpret_cast<const u32x4_t *>(ptr) : u32x4_t{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int h = hb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
                w[hb][r] = h < H ? a.W[(size_t)t * H + h] : 0.f;
            }
        }
    }

    // FP8 scoring: each (query, head) row is quantized to e4m3fn with its own
    // scale amax / 448 (round to nearest even; |q| / scale <= 448 is finite),
    // and the scale is folded into the head weight, which is exact to fp32
    // rounding because ReLU commutes with a positive factor:
    //   w * ReLU(q . k) ~= (w * scale) * ReLU((q / scale) . k).
    // Lane l holds head l % 32 and the 32 elements 64 kk + 32 (l / 32) of each
    // k-step; the B fragments of the keys use the same element order.
    __device__ void load_q8(const FusedArgs &a, int t)
    {
        const int l = (int)lane_id();
        const int H = a.H;
        const int half = l >> 5;
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) {
            const int head = hb * 32 + (l & 31);
            const bool ok = head < H;
            float x[C::KS][32];
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                const int d0 = kk * 64 + 32 * half;
                const char *ptr = static_cast<const char *>(a.Q) + (((size_t)t * H + (ok ? head : 0)) * C::D + d0) * 2;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4_t v = ok ? *reinterpret_cast<const u32x4_t *>(ptr + 16 * c) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wd = v[e];
                        if constexpr (C::QT == ITK_BF16) {
                            x[kk][8 * c + 2 * e] = __uint_as_float(wd << 16);
                            x[kk][8 * c + 2 * e + 1] = __uint_as_float(wd & 0xFFFF0000u);
                        } else {
                            x[kk][8 * c + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFFu));
                            x[kk][8 * c + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
                        }
                    }
                }
            }
            float amax = 0.f;
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
                for (int i = 0; i < 32; ++i) amax = fmaxf(amax, __builtin_fabsf(x[kk][i]));
            // lanes l and l ^ 32 hold the two halves of the same row
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
            amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            const bool pos = amax > 0.f && __builtin_isfinite(amax);
            const float inv = pos ? 448.f / amax : 0.f;
            const float qs = pos ? amax / 448.f : 1.f;
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                u32x8_t f;
#pragma unroll
                for (int wd = 0; wd < 8; ++wd) {
                    int v = 0;
                    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[kk][4 * wd] * inv, x[kk][4 * wd + 1] * inv, v, false);
                    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[kk][4 * wd + 2] * inv, x[kk][4 * wd + 3] * inv, v, true);
                    f[wd] = (uint32_t)v;
                }
                q[hb][kk] = f;
            }
            // weights of the accumulator rows this lane holds, times their rows' scales
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int h = hb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const float sc = __shfl(qs, h & 31);
                w[hb][r] = h < H ? a.W[(size_t)t * H + h] * sc : 0.f;
            }
        }
    }

    // Make the loaded fragments resident before a loop that uses them.  The
    // waits for these loads then sit here, once, instead of inside the loop
    // where they would also wait for that loop's own prefetches.
    __device__ __forceinline__ void settle()
    {
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) {
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) asm volatile("" : "+v"(q[hb][kk]));
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(w[hb][r]));
        }
    }
};

// ReLU of an fp32 value as one integer max: negative values (sign bit set,
// including -0) compare below 0 as int32 and become +0; positive values keep
// their bits.  Unlike fmaxf it needs no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// Head reduction of one 32-key block: lane l sums w * ReLU(acc) over the 16
// head rows it holds in each 32-head block, for key column l % 32.  The two
// half-waves hold disjoint head rows of the same keys.
template <class C>
__device__ __forceinline__ float reduce_block(const f32x16_t (&acc)[C::HB], const float (&w)[C::HB][16])
{
    float s = 0.f;
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = acc[hb][r];
            s = fmaf(w[hb][r], C::RELU ? relu_bits(x) : x, s);
        }
    return s;
}

// Combine the half-wave partials of two consecutive 32-key blocks so that
// lane l holds the score of key l of the 64-key tile: v_permlane32_swap
// exchanges the upper half of p0 with the lower half of p1, after which
// lane l < 32 holds p0[l] and p0[l + 32] and lane l >= 32 holds p1[l - 32]
// and p1[l].
__device__ __forceinline__ float combine_halves(float p0, float p1)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMAs of one 32-key block of a staged 64-key tile into acc.  `bl` is the
// lane's byte address of its first B fragment in the block: lane l supplies
// key column l % 32 at the k-slice selected by l / 32 (bf16/fp16: 8 values
// at element 8 (l / 32) of each 16-element step; fp32: element l / 32 of each
// 2-element step).  The B fragments are read from LDS in chunks of KCH
// k-steps, at compile-time offsets from `bl`.
template <class C>
__device__ __forceinline__ void block_mfma(f32x16_t (&acc)[C::HB], const QFrags<C> &qf, const char *bl)
{
    constexpr int KCH = C::KS < 8 ? C::KS : 8;
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) acc[hb] = f32x16_t{};
#pragma unroll
    for (int k0 = 0; k0 < C::KS; k0 += KCH) {
        typename C::frag b[KCH];
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int kk = k0 + i;
            if constexpr (C::MT == M_F32)
                b[i] = *reinterpret_cast<const float *>(bl + kk * 8);
            else if constexpr (C::MT == M_FP8)
                b[i] = *reinterpret_cast<const u32x8_t *>(bl + kk * 64);
            else
                b[i] = *reinterpret_cast<const u32x4_t *>(bl + kk * 32);
        }
#pragma unroll
        for (int i = 0; i < KCH; ++i)
#pragma unroll
            for (int hb = 0; hb < C::HB; ++hb) acc[hb] = mfma32<C::MT>(qf.q[hb][k0 + i], b[i], acc[hb]);
    }
}

// Byte offset of lane l's first B fragment within a staged 64-key tile.
template <class C>
__device__ __forceinline__ int bfrag_lane_off()
{
    const int l = (int)lane_id();
    return (l & 31) * C::ROWP + (C::MT == M_F32 ? (l >> 5) * 4 : C::MT == M_FP8 ? (l >> 5) * 32 : (l >> 5) * 16);
}

// Scheduling hint for one block: per chunk, the B-fragment LDS reads, then
// every MFMA followed by a few VALU instructions of the previous block's head
// reduction, so that the reduction issues while the matrix core works.
template <class C>
__device__ __forceinline__ void sched_block()
{
    constexpr int KCH = C::KS < 8 ? C::KS : 8;
    constexpr int NM = C::KS * C::HB;
    constexpr int NV = 32 * C::HB;  // max + fma per accumulator register
    constexpr int PER = (NV + NM - 1) / NM;
#pragma unroll
    for (int k0 = 0; k0 < C::KS; k0 += KCH) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < KCH * C::HB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
        }
    }
}

// B fragments of one 32-key block read straight from global K (recovery
// route and the few-query scan): lane l holds key column l % 32 at the
// k-slice l / 32 of every k-step.  All of a block's loads are issued by
// load() before any is used; FP8 keys are kept as loaded and widened (like
// the staged copy) only in score(), so that load() never waits for data.
template <class C>
struct GlobalBlock {
    static constexpr bool WIDEN = C::KT == ITK_FP8_E4M3 && C::MT != M_FP8;
    typename C::frag b[WIDEN ? 1 : C::KS];
    u32x2_t raw[WIDEN ? C::KS : 1];
    // bytes per lane that a block's loads hold
    static constexpr int BYTES = WIDEN ? C::KS * 8 : C::KS * (int)sizeof(typename C::frag);
    __device__ __forceinline__ void load(const FusedArgs &a, int64_t kb0)
    {
        const int l = (int)lane_id();
        const int64_t key = kb0 + (l & 31);
        const bool ok = key < a.N;
        const char *krow = static_cast<const char *>(a.K) + (size_t)(ok ? key : 0) * C::D * C::kbytes;
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            if constexpr (C::MT == M_F32) {
                b[kk] = ok ? reinterpret_cast<const float *>(krow)[kk * 2 + (l >> 5)] : 0.f;
            } else if constexpr (C::MT == M_FP8) {
                const int d0 = kk * 64 + 32 * (l >> 5);
                b[kk] = ok ? *reinterpret_cast<const u32x8_t *>(krow + d0) : u32x8_t{};
            } else if constexpr (WIDEN) {
                const int d0 = kk * 16 + 8 * (l >> 5);
                raw[kk] = ok ? *reinterpret_cast<const u32x2_t *>(krow + d0) : u32x2_t{0u, 0u};
            } else {
                const int d0 = kk * 16 + 8 * (l >> 5);
                b[kk] = ok ? *reinterpret_cast<const u32x4_t *>(krow + d0 * 2) : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }
    // The block's weighted, ReLU'd head sum per lane (half of a key's score).
    __device__ __forceinline__ float score(const QFrags<C> &qf) const
    {
        f32x16_t acc[C::HB];
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) acc[hb] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            typename C::frag f;
            if constexpr (WIDEN) {
                const u32x2_t lo = fp8x4_widen<C::MT>(raw[kk][0]), hi = fp8x4_widen<C::MT>(raw[kk][1]);
                f = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            } else {
                f = b[kk];
            }
#pragma unroll
            for (int hb = 0; hb < C::HB; ++hb) acc[hb] = mfma32<C::MT>(qf.q[hb][kk], f, acc[hb]);
        }
        return reduce_block<C>(acc, qf.w);
    }
};

// Same scores with B fragments read straight from global K (recovery path).
// One block's fragments are live at a time (the select kernel that runs it
// has little register room).
template <class C>
__device__ float tile_scores_global(const QFrags<C> &qf, const FusedArgs &a, int64_t key0)
{
    GlobalBlock<C> gb;
    gb.load(a, key0);
    const float p0 = gb.score(qf);
    gb.load(a, key0 + 32);
    const float p1 = gb.score(qf);
    return combine_halves(p0, p1);
}

// ---------------------------------------------------- tile staging (LDS)
// Double-buffered key stages (and the per-key scales of FP8 keys).
template <class C, int NS = C::NSUB>
struct TileBuf {  // NS 64-key tiles per stage
    char k[2][NS * C::TILE_LDS];
    float scale[2][C::SCALE ? NS * TILE_KEYS : 1];
};

// Per-key FP8 scales of a stage whose key bytes are copied straight to LDS:
// thread i < NSUB * 64 loads the scale of key i of the stage into a register
// when the stage's copy is issued, and stores it to LDS after the copy's wait.
template <class C, int NSUB>
struct ScaleStage {
    float v = 1.f;
    __device__ __forceinline__ void load(const FusedArgs &a, int64_t key0)
    {
        const int64_t key = key0 + (int64_t)threadIdx.x;
        if (threadIdx.x < NSUB * TILE_KEYS) v = key < a.N ? a.k_scale[key] : 0.f;
    }
    template <class TB>
    __device__ __forceinline__ void store(TB &tb, int buf) const
    {
        if (threadIdx.x < NSUB * TILE_KEYS) tb.scale[buf][threadIdx.x] = v;
    }
};

// One wave instruction of the direct global -> LDS copy: lane i's 16 bytes
// at byte `voff` from the wave-uniform address `sbase` land at LDS byte
// lds_base + 16 i (lds_base is wave-uniform and goes through M0, which is
// restored afterwards).  Issued from inline assembly so that the compiler
// does not fence later LDS accesses of other buffers on it; the caller waits
// for completion (vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void lds_dma16(const void *sbase_in, uint32_t voff, uint32_t lds_base)
{
    // the address is wave-uniform by construction; say so to the compiler
    // (readfirstlane returns int: go through uint32_t, or the low word would
    // be sign-extended into the high one)
    const uint64_t sb = (uint64_t)sbase_in;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
    const void *sbase = (const void *)(((uint64_t)hi << 32) | (uint64_t)lo);
    lds_base = (uint32_t)__builtin_amdgcn_readfirstlane(lds_base);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory");
}

template <class T>
__device__ __forceinline__ uint32_t lds_addr(T *p)
{
    return (uint32_t)(size_t)(__attribute__((address_space(3))) char *)p;
}

// Direct global -> LDS copy of a stage of NSUB * 64 keys.  The stage's LDS
// image is NSUB * 64 * SPR 16-byte slots, copied in 1 KB pieces (one wave
// instruction each: lane i writes slot 64 j + i of piece j); piece j goes to
// wave j % 8.  Slot q holds chunk q % SPR of row q / SPR; the pad slot of a
// row re-reads the row's first chunk.  The per-lane source offsets within
// the stage are fixed, so they are computed once (DmaPlan); keys past N
// re-read key N-1 (their scores are never used).
template <class C, int NSUB>
struct DmaPlan {
    static constexpr int PIECES = NSUB * TILE_KEYS * C::SPR / 64;
    static constexpr int PER_WAVE = (PIECES + FUSED_WAVES - 1) / FUSED_WAVES;
    static_assert(PIECES * 64 == NSUB * TILE_KEYS * C::SPR, "stage must split into 1 KB pieces");
    static_assert((C::ROWB & (C::ROWB - 1)) == 0, "key rows are a power of two bytes");
    uint32_t src_off[PER_WAVE];  // row * ROWB + chunk * 16, from the stage's first key

    __device__ void init()
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int q = (j * FUSED_WAVES + wave) * 64 + lane;
            const int r = q / C::SPR, c = q % C::SPR;
            src_off[j] = (uint32_t)(r * C::ROWB + (c < C::CH ? c : 0) * 16);
        }
    }

    // Copies the stage starting at key0 into buffer `buf`.  Rows at or past
    // key N re-read the same chunk of the last key (never read back).
    template <class TB>
    __device__ __forceinline__ void issue(const FusedArgs &a, TB &tb, int buf, int64_t key0) const
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t base = lds_addr(tb.k[buf]);
        const char *kbase = static_cast<const char *>(a.K) + (size_t)key0 * C::ROWB;
        const bool tail = key0 + NSUB * TILE_KEYS > a.N;
        const uint32_t last_row = (uint32_t)(a.N - 1 - key0);  // key0 < N
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int piece = j * FUSED_WAVES + wave;
            if (piece < PIECES) {
                uint32_t off = src_off[j];
                if (tail) {
                    const uint32_t r = off / C::ROWB;
                    off = (r < last_row ? r : last_row) * C::ROWB + (off & (C::ROWB - 1));
                }
                lds_dma16(kbase, off, base + (uint32_t)piece * 1024u);
            }
        }
    }
};

// FP8 staging through registers: each of the FUSED_THREADS threads moves
// EPT consecutive elements of one key of a 64-key tile (thread -> key tid/8,
// part tid%8), widening them to the MFMA operand type; threads 0..63 also
// move the tile's per-key scales.
template <class C>
struct KStage {
    static constexpr int RB = C::EPT * C::kbytes;  // raw bytes per thread
    static_assert(!C::SCALE || RB == 8 || RB == 16 || RB == 32, "unsupported FP8 staging width");
    static constexpr int NW = C::SCALE ? RB / 4 : 2;
    uint32_t words[NW];
    float sc;

    __device__ void load(const FusedArgs &a, int64_t key0)
    {
        const int tid = threadIdx.x;
        const int64_t key = key0 + (tid >> 3);
        const int part = tid & 7;
        const bool ok = key < a.N;
        const char *src = static_cast<const char *>(a.K) + ((size_t)(ok ? key : 0) * C::D + part * C::EPT) * C::kbytes;
#pragma unroll
        for (int i = 0; i < NW; i += 2) {
            const u32x2_t v = ok ? reinterpret_cast<const u32x2_t *>(src)[i / 2] : u32x2_t{0u, 0u};
            words[i] = v[0];
            words[i + 1] = v[1];
        }
        if (tid < TILE_KEYS) {
            const int64_t ks = key0 + tid;
            sc = ks < a.N ? a.k_scale[ks] : 0.f;
        }
    }

    template <class TB>
    __device__ void store(TB &tb, int buf) const
    {
        const int tid = threadIdx.x;
        const int r = tid >> 3, part = tid & 7;
        // EPT fp8 values -> EPT 16-bit values = EPT / 8 chunks of 16 bytes
#pragma unroll
        for (int o = 0; o < C::EPT / 8; ++o) {
            const u32x2_t lo = fp8x4_widen<C::MT>(words[o * 2]), hi = fp8x4_widen<C::MT>(words[o * 2 + 1]);
            const int c = part * (C::EPT / 8) + o;
            *reinterpret_cast<u32x4_t *>(tb.k[buf] + r * C::ROWP + c * 16) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
        if (tid < TILE_KEYS) tb.scale[buf][tid] = sc;
    }
};

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

// The pipelined tile scan shared by the sample and main passes.
//
// Visits `nstages` stages of NSUB consecutive 64-key tiles, the first at key
// `first` and each `step` keys after the previous one; tiles at or beyond
// `key_end` are skipped.  The workgroup stages each stage once into LDS
// (double-buffered: the next stage's copy is in flight during the current
// stage's compute); each wave whose query still has valid keys in a tile
// scores it against its own query.  A tile is split into two 32-key blocks
// with separate accumulators, and every block's MFMAs are issued interleaved
// with the VALU head reduction of the block before it, so matrix and vector
// work of one wave overlap.  A tile's scores are therefore complete one block
// later; visit(key0, s) is called once per scored tile (wave-uniform) with
// lane l holding the score of key key0 + l (scaled by the per-key FP8 scale),
// which the visitor must mask against the query's length.  Every thread of
// the workgroup must call this.
// Per-stage hook of scan_tiles: issue() runs just before the wait for the
// next stage's copy (a load it issues completes with that wait), use() just
// after the stage barrier.
struct NoStageHook {
    __device__ __forceinline__ void issue() {}
    __device__ __forceinline__ void use() {}
};

template <class C, int NSUB, class TB, class Visit, class Hook = NoStageHook>
__device__ __forceinline__ void scan_tiles(const FusedArgs &a, TB &tb, const QFrags<C> &qf, int64_t first,
                                           int64_t step, int nstages, int64_t key_end, bool active, uint32_t L,
                                           Visit &&visit, Hook &&hook = Hook{})
{
    static_assert(C::DMA || NSUB == 1, "FP8 staging moves one 64-key tile per stage");
    static_assert(sizeof(tb.k[0]) >= NSUB * C::TILE_LDS, "stage buffer too small");
    const int lane = (int)lane_id();
    const int64_t kend = key_end < (int64_t)L ? key_end : (int64_t)L;
    KStage<C> ks;
    DmaPlan<C, NSUB> dp;
    ScaleStage<C, NSUB> ss;
    constexpr bool DSCALE = C::DMA && C::SCALE;  // scales beside copied FP8 key bytes
    if constexpr (C::DMA) dp.init();
    if (nstages > 0) {
        if constexpr (C::DMA) {
            dp.issue(a, tb, 0, first);
            if constexpr (DSCALE) ss.load(a, first);
        } else {
            ks.load(a, first);
            ks.store(tb, 0);
        }
    }
    const_cast<QFrags<C> &>(qf).settle();
    wait_vmem_all();
    if constexpr (DSCALE) ss.store(tb, 0);
    __syncthreads();
    f32x16_t accA[C::HB], accB[C::HB];
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) {
        accA[hb] = f32x16_t{};
        accB[hb] = f32x16_t{};
    }
    float p0 = 0.f, psc = 1.f;
    int64_t pend = -1;  // key0 of the tile whose block 1 sits in accB
    const int boff = bfrag_lane_off<C>();
    for (int st = 0; st < nstages; ++st) {
        const int64_t skey = first + (int64_t)st * step;
        const int buf = st & 1;
        if (st + 1 < nstages) {
            if constexpr (C::DMA) {
                dp.issue(a, tb, buf ^ 1, skey + step);
                if constexpr (DSCALE) ss.load(a, skey + step);
            } else {
                ks.load(a, skey + step);
            }
        }
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
            const int64_t key0 = skey + sub * TILE_KEYS;
            if (active && key0 < kend) {
                const char *bl = tb.k[buf] + boff + sub * C::TILE_LDS;
                // block 0 of this tile, overlapped with the reduction of
                // block 1 of the previous one
                block_mfma<C>(accA, qf, bl);
                float p1 = reduce_block<C>(accB, qf.w);
                sched_block<C>();
                asm volatile("" : "+v"(p1));  // keep the reduction in this region
                if (pend >= 0) visit(pend, combine_halves(p0, p1) * psc);
                // block 1, overlapped with the reduction of block 0
                block_mfma<C>(accB, qf, bl + 32 * C::ROWP);
                p0 = reduce_block<C>(accA, qf.w);
                sched_block<C>();
                asm volatile("" : "+v"(p0));
                if constexpr (C::SCALE) psc = tb.scale[buf][sub * TILE_KEYS + lane];
                pend = key0;
            } else if (pend >= 0) {
                const float p1 = reduce_block<C>(accB, qf.w);
                visit(pend, combine_halves(p0, p1) * psc);
                pend = -1;
            }
        }
        if (st + 1 < nstages) {
            if constexpr (!C::DMA) ks.store(tb, buf ^ 1);
            hook.issue();
            wait_vmem_all();
            if constexpr (DSCALE) ss.store(tb, buf ^ 1);
        }
        __syncthreads();
        if (st + 1 < nstages) hook.use();
    }
    if (pend >= 0) {
        const float p1 = reduce_block<C>(accB, qf.w);
        visit(pend, combine_halves(p0, p1) * psc);
    }
}

// Wave-level search: the largest bin b with sum_{b' >= b} hist[b'] >= q,
// or -1 when the histogram holds fewer than q items.  Lane l owns bins
// [NBINS - 32(l+1), NBINS - 32 l).
template <class HistPtr>
__device__ int wave_top_bin(HistPtr hist, uint32_t q)
{
    const int l = (int)lane_id();
    const int hi = NBINS - 32 * l;  // exclusive
    uint32_t c[32];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        c[i] = hist[hi - 1 - i];
        s += c[i];
    }
    const uint32_t incl = wave_incl_sum(s);
    const uint64_t m = __ballot(incl >= q);
    if (!m) return -1;
    const int f = __ffsll((unsigned long long)m) - 1;
    int bin = 0;
    if (l == f) {
        uint32_t cum = incl - s;
        bin = hi - 32;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (cum + c[i] >= q) { bin = hi - 1 - i; break; }
            cum += c[i];
        }
    }
    return (int)lane_value((uint32_t)bin, f);
}

// Keys of sampled tile number `m` (0-based within the split's sampled tiles).
struct SampleIter {
    int64_t first_key;  // key of the first sampled tile in the split, or -1
    int64_t stride_keys;
    int64_t end;        // exclusive key bound for the split
    int ntiles;
};
__device__ __forceinline__ SampleIter sample_iter(const FusedArgs &a, int g, int p, uint32_t maxL)
{
    SampleIter it;
    const int64_t st = a.sample_tiles, phase = g % a.sample_tiles;
    const int64_t lo = (int64_t)p * a.span_s;
    int64_t hi = lo + a.span_s;
    if (hi > (int64_t)maxL) hi = maxL;
    it.stride_keys = st * TILE_KEYS;
    it.end = hi;
    const int64_t t0 = lo / TILE_KEYS;  // first tile of the split (lo is tile aligned)
    int64_t first = t0 + ((phase - t0 % st) % st + st) % st;
    it.first_key = first * TILE_KEYS < hi ? first * TILE_KEYS : -1;
    it.ntiles = it.first_key >= 0 ? (int)((hi - it.first_key + it.stride_keys - 1) / it.stride_keys) : 0;
    return it;
}

__device__ __forceinline__ uint32_t group_max_len(const FusedArgs &a, int g)
{
    uint32_t m = 0;
    for (int w = 0; w < FUSED_WAVES; ++w) {
        const int t = g * FUSED_WAVES + w;
        if (t < a.T) {
            const uint32_t L = kv_length(a, t);
            m = L > m ? L : m;
        }
    }
    return m;
}

// ------------------------------------------- history sample: gather rows
// Entry e < n_prior of the caller's list names key prior[e]; entries outside
// [0, N) (and the padding up to whole tiles) are unusable.  Each thread moves
// one 16-byte chunk of an entry's key row into the gathered copy, which the
// sample passes then scan like K; unusable entries get a zero row and the
// index INT32_MAX, which no row's length exceeds.
template <class C>
__global__ __launch_bounds__(256) void k_prior_gather(FusedArgs a)
{
    constexpr int ch = C::D * C::kbytes / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t e = gid / ch;
    const int c = (int)(gid - e * ch);
    if (e >= a.np) return;
    const int64_t j = e < a.n_prior ? (int64_t)a.prior[e] : -1;
    const bool ok = j >= 0 && j < a.N;
    const u32x4_t v = ok ? *reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.K) + j * a.rowb + c * 16)
                         : u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t *>(static_cast<char *>(a.Kp) + e * a.rowb + c * 16) = v;
    if (c == 0) {
        a.pidx[e] = ok ? (int32_t)j : 0x7FFFFFFF;
        if (a.kp_scale) a.kp_scale[e] = ok ? a.k_scale[j] : 0.f;
    }
}

// -------------------------------------------- sample pass A: score range
// PRIOR: the history sample.  The scan then runs over the gathered entries
// (their key rows stand in for K) in stages of the main scan's size (the
// entries of a split are contiguous tiles), and entry e is usable for the row
// when its key is below the row's length.  A separate instantiation, so that
// the strided view keeps its own register allocation.
template <class C, bool PRIOR>
__global__ __launch_bounds__(FUSED_THREADS) void k_fused_minmax(FusedArgs a)
{
    constexpr int NS = PRIOR ? C::NSUB : 1;  // 64-key tiles per stage
    __shared__ TileBuf<C, NS> tb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int g, p;
    map_group_split(blockIdx.x, a.G, a.Ps, g, p);
    const int t = g * FUSED_WAVES + wave;
    const bool active = t < a.T;
    const uint32_t L = active ? kv_length(a, t) : 0u;
    if (p == 0 && active) {  // per-call reset of the row's counters
        for (int i = lane; i < NBINS; i += 64) {
            a.hist[(size_t)t * NBINS + i] = 0u;
            a.hist_r[(size_t)t * NBINS + i] = 0u;
        }
        if (lane == 0) {
            a.tail[t] = 0u;
            a.rflag[t] = 0u;
            a.gpub[t] = 0u;
            if (PRIOR) a.pcount[t] = 0u;
        }
    }
    FusedArgs sa = a;
    if (PRIOR) {
        sa.K = a.Kp;
        sa.k_scale = a.kp_scale;
        sa.N = a.np;
    }
    const uint32_t maxL = PRIOR ? (uint32_t)a.np : group_max_len(a, g);
    const SampleIter it = sample_iter(a, g, p, maxL);
    QFrags<C> qf;
    if (active) qf.load(a, t);
    float mn = __builtin_inff(), mx = -__builtin_inff();
    // When the plan gives room for it, the view's scores are also stored
    // (sampled tile j of the row at samp[t][64 j ...], NaN past the row), so
    // that pass B bins them without scoring the view again.
    const int64_t phase = g % a.sample_tiles;
    float *srow = a.samp ? a.samp + (size_t)(active ? t : 0) * a.samp_cap : nullptr;
    const uint32_t Lscan = PRIOR ? (uint32_t)a.np : L;
    const int64_t step = PRIOR ? (int64_t)NS * TILE_KEYS : it.stride_keys;
    const int nst = PRIOR ? (it.ntiles + NS - 1) / NS : it.ntiles;
    scan_tiles<C, NS>(sa, tb, qf, it.first_key, step, nst, it.end, active, Lscan, [&](int64_t key0, float s) {
        const bool valid = PRIOR ? a.pidx[key0 + lane] < (int32_t)L : key0 + lane < (int64_t)L;
        if (valid) {
            mn = fminf(mn, s);
            mx = fmaxf(mx, s);
        }
        if (srow) srow[((key0 / TILE_KEYS - phase) / a.sample_tiles) * TILE_KEYS + lane] = valid ? s : __builtin_nanf("");
    });
    if (active) {
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane == 0) a.mm[(size_t)t * a.Ps + p] = make_float2(mn, mx);
    }
}

// Equal-width bin mapping from the sampled score range (m = NBINS bins).
// Called by every lane of a wave: the Ps per-split ranges are read by the
// lanes in parallel (a one-query decode call has 256 splits; read one after
// the other they took most of the histogram pass).
__device__ __forceinline__ float4 bin_params(const FusedArgs &a, int t)
{
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int p = (int)lane_id(); p < a.Ps; p += 64) {
        const float2 v = a.mm[(size_t)t * a.Ps + p];
        mn = fminf(mn, v.x);
        mx = fmaxf(mx, v.y);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    const float delta = (float)NBINS / (mx - mn);
    const bool ok = (mx > mn) && __builtin_isfinite(delta) && delta > 0.f && __builtin_isfinite(mn);
    return ok ? make_float4(-mn * delta, delta, 0.f, 0.f) : make_float4(0.f, 0.f, 1.f, 0.f);
}

__device__ __forceinline__ uint32_t bin_of(float b)
{
    return (uint32_t)fminf(fmaxf(floorf(b), 0.f), (float)(NBINS - 1));
}

// ---------------------------------------- sample pass B: sample histogram
// Bins the view scores that pass A stored (the same tiles of the same split,
// so every score is counted once), or, when the plan stores no view (a view
// larger than the candidate buffer), scores the view again.
// STORED: pass A stored the sampled scores (the planner decides), so this
// pass only reads them; the other instantiation scores the sample again.
// Separate instantiations, so that the reading one carries neither the
// scoring registers nor the key stages.
template <class C, bool STORED>
__global__ __launch_bounds__(FUSED_THREADS) void k_fused_samplehist(FusedArgs a)
{
    __shared__ uint32_t whist[FUSED_WAVES][NBINS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int g, p;
    map_group_split(blockIdx.x, a.G, a.Ps, g, p);
    const int t = g * FUSED_WAVES + wave;
    const bool active = t < a.T;
    const uint32_t L = active ? kv_length(a, t) : 0u;
    for (int i = lane; i < NBINS; i += 64) whist[wave][i] = 0u;
    float4 bp = make_float4(0.f, 0.f, 1.f, 0.f);
    if (active) {
        bp = bin_params(a, t);
        if (p == 0 && lane == 0) a.param[t] = bp;
    }
    const bool prior = a.pidx != nullptr;
    const uint32_t maxL = prior ? (uint32_t)a.np : group_max_len(a, g);
    const SampleIter it = sample_iter(a, g, p, maxL);
    // a degenerate sampled range leaves the gate open: nothing to count
    const bool count = active && bp.z == 0.f;
    if constexpr (!STORED) {
        __shared__ TileBuf<C, 1> tb;
        QFrags<C> qf;
        if (active) qf.load(a, t);
        scan_tiles<C, 1>(a, tb, qf, it.first_key, it.stride_keys, it.ntiles, it.end, count, L,
                         [&](int64_t key0, float s) {
                             if (key0 + lane < (int64_t)L) atomicAdd(&whist[wave][bin_of(fmaf(s, bp.y, bp.x))], 1u);
                         });
    } else if (count) {
        // the tiles pass A visited: first_key + i * stride below min(end, L)
        // (a history sample stores every entry of the split, NaN where unusable)
        const int64_t kend = prior || it.end < (int64_t)L ? it.end : (int64_t)L;
        const int64_t phase = g % a.sample_tiles;
        const float *srow = a.samp + (size_t)t * a.samp_cap;
        int n = 0;
        if (it.first_key >= 0 && it.first_key < kend)
            n = (int)((kend - it.first_key + it.stride_keys - 1) / it.stride_keys);
        if (n > it.ntiles) n = it.ntiles;
        const int64_t j0 = (it.first_key / TILE_KEYS - phase) / a.sample_tiles;  // first sampled tile's slot
        constexpr int B = 8;  // loads in flight per lane
        uint32_t usable = 0;
        for (int i0 = 0; i0 < n; i0 += B) {
            float v[B];
#pragma unroll
            for (int j = 0; j < B; ++j)
                v[j] = i0 + j < n ? srow[(j0 + i0 + j) * TILE_KEYS + lane] : __builtin_nanf("");
#pragma unroll
            for (int j = 0; j < B; ++j)
                if (v[j] == v[j]) {
                    atomicAdd(&whist[wave][bin_of(fmaf(v[j], bp.y, bp.x))], 1u);
                    ++usable;
                }
        }
        if (prior) {
            usable = lane_value(wave_incl_sum(usable), 63);
            if (lane == 0 && usable) atomicAdd(&a.pcount[t], usable);
        }
    }
    __syncthreads();
    if (count) {
        for (int i = lane; i < NBINS; i += 64) {
            const uint32_t c = whist[wave][i];
            if (c) atomicAdd(&a.hist[(size_t)t * NBINS + i], c);
        }
    }
}

// ------------------------------------------------ main pass: filter scan

template <class C>
__global__ __launch_bounds__(FUSED_THREADS) void k_fused_main(FusedArgs a)
{
    // Separate LDS objects, so that the compiler can tell the histogram and
    // staging accesses apart from the in-flight key-tile copies.
    __shared__ TileBuf<C> tb;
    __shared__ uint32_t whist_all[FUSED_WAVES][NBINS];
    __shared__ Cand stage_all[FUSED_WAVES][128];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int g, p;
    map_group_split(blockIdx.x, a.G, a.P, g, p);
    if (a.force == 1) return;  // every row takes the recovery route (the sample still sets its bins)
    const int t = g * FUSED_WAVES + wave;
    const bool active = t < a.T;
    const uint32_t L = active ? kv_length(a, t) : 0u;
    const uint32_t maxL = group_max_len(a, g);
    const int64_t k_lo = (int64_t)p * a.span;
    int64_t k_hi = k_lo + a.span;
    if (k_hi > (int64_t)maxL) k_hi = maxL;
    const int nstages = k_hi > k_lo ? (int)((k_hi - k_lo + C::STAGE_KEYS - 1) / C::STAGE_KEYS) : 0;

    uint32_t *whist = whist_all[wave];
    Cand *stage = stage_all[wave];
    for (int i = lane; i < NBINS; i += 64) whist[i] = 0u;

    // Initial threshold bin from the sample (wave-uniform state).
    float off = 0.f, delta = 0.f;
    int gate_bin = 0;
    float gate_f = -__builtin_inff();
    if (active) {
        const float4 bp = a.param[t];
        const RowSample rs = row_sample(a, t, g, L, bp.z != 0.f);
        if (!rs.admit_all) {
            off = bp.x;
            delta = bp.y;
            const int b = wave_top_bin(a.hist + (size_t)t * NBINS, rs.q0);
            gate_bin = b > 0 ? b : 0;
            gate_f = gate_bin > 0 ? (float)gate_bin : -__builtin_inff();
        }
    }
    QFrags<C> qf;
    if (active) qf.load(a, t);
    // Threshold refresh state (wave-uniform): `inrange` counts the admitted
    // keys whose bin is >= gate_bin, `at_gate` those whose bin == gate_bin.
    // Whenever the keys strictly above the gate bin number at least k, every
    // key of the row's Top-k lies above it too, so the gate moves up a bin
    // (LiteTopK Sec. 3.2: the threshold is the bin holding the k-th largest
    // score seen so far).
    uint32_t stage_n = 0, inrange = 0, at_gate = 0;
    uint32_t tail_reg = 0;  // candidate count when this wave owns the whole row
    const bool own_row = a.P == 1;
    Cand *cand = a.cand + (size_t)(active ? t : 0) * a.cap;
    const uint32_t cap = (uint32_t)a.cap;
    const uint32_t kq = (uint32_t)a.k;
    const bool refresh = delta > 0.f;

    auto flush = [&](uint32_t n) {
        uint32_t slot = 0;
        if (own_row) {
            slot = tail_reg;
            tail_reg += n;
        } else {
            if (lane == 0) slot = atomicAdd(&a.tail[t], n);
            slot = lane_value(slot, 0);
        }
        if ((uint32_t)lane < n && slot + lane < cap) cand[slot + lane] = stage[lane];
    };
    // Moves the gate up to bin nb (<= NBINS - 1), keeping the counts.
    auto raise_to = [&](int nb) __attribute__((always_inline)) {
        while (gate_bin < nb) {
            inrange -= at_gate;
            ++gate_bin;
            at_gate = whist[gate_bin];
        }
        gate_f = (float)gate_bin;
    };
    // Under key splits each split refreshes its gate from its own admitted
    // keys; a split whose own keys put the gate above a bin proves that every
    // key of the row's Top-k lies above it (LiteTopK Sec. 3.2), so the bin is
    // published to the row's word (atomic max) and the other splits of the
    // row read it once per stage, with the stage's copy, and move up to it.
    const bool publish = !own_row && active && refresh;
    struct PubHook {
        const FusedArgs &a;
        int t;
        bool on;
        uint32_t v;
        decltype(raise_to) &raise;
        const int &cur;
        __device__ __forceinline__ void issue()
        {
            if (on) v = a.gpub[t];
        }
        __device__ __forceinline__ void use()
        {
            if (on) {
                const int pub = (int)__builtin_amdgcn_readfirstlane(v);
                if (pub > cur) raise(pub < NBINS - 1 ? pub : NBINS - 1);
            }
        }
    } hook{a, t, publish, 0u, raise_to, gate_bin};

    scan_tiles<C, C::NSUB>(a, tb, qf, k_lo, C::STAGE_KEYS, nstages, k_hi, active, L, [&](int64_t key0, float s) {
        const int64_t key = key0 + lane;
        const bool valid = key < (int64_t)L;
        const float b = fmaf(s, delta, off);
        const bool pass = valid && b >= gate_f;
        const uint64_t m = __ballot(pass);
        if (m) {
            const uint32_t bin = bin_of(b);
            const uint32_t pos = stage_n + lanes_below(m);
            if (pass) {
                atomicAdd(&whist[bin], 1u);
                stage[pos] = Cand{(uint32_t)key, s};
            }
            const uint32_t n = (uint32_t)__popcll(m);
            stage_n += n;
            inrange += n;
            at_gate += (uint32_t)__popcll(__ballot(pass && bin == (uint32_t)gate_bin));
            if (stage_n >= 64u) {
                flush(64u);
                const bool mv = (uint32_t)lane < stage_n - 64u;
                Cand e;
                if (mv) e = stage[64 + lane];
                if (mv) stage[lane] = e;
                stage_n -= 64u;
            }
            if (refresh && inrange - at_gate >= kq && gate_bin < NBINS - 1) {
                do {
                    inrange -= at_gate;
                    ++gate_bin;
                    at_gate = whist[gate_bin];
                } while (inrange - at_gate >= kq && gate_bin < NBINS - 1);
                gate_f = (float)gate_bin;
                if (publish && lane == 0) atomicMax(&a.gpub[t], (uint32_t)gate_bin);
            }
        }
    }, hook);
    if (active && stage_n) flush(stage_n);
    if (active && own_row && lane == 0) a.tail[t] = tail_reg;
}

// One 32-key block copied by one wave into its own LDS rows (few-query
// scan): each load instruction reads whole 16-byte chunks of consecutive key
// rows (RC lanes per row), so the global reads are coalesced; store() writes
// them (FP8 keys widened) into the padded row layout of the staged tiles, so
// that block_mfma reads the B fragments as in the staged scan.
template <class C>
struct WaveBlock {
    static constexpr int RAW = C::D * C::kbytes;  // global bytes per key row
    static constexpr int RC = RAW / 16;           // 16-byte chunks per row
    static constexpr int RPI = 64 / RC;           // rows per load instruction
    static constexpr int NI = 32 / RPI;           // load instructions per block
    static constexpr bool WIDEN = C::KT == ITK_FP8_E4M3 && C::MT != M_FP8;
    static constexpr bool OK = RC >= 1 && RC <= 16 && 64 % RC == 0 && 32 * C::ROWP * FUSED_WAVES <= 80 * 1024;
    u32x4_t v[OK ? NI : 1];
    __device__ __forceinline__ void load(const FusedArgs &a, int64_t kb0)
    {
        const int l = (int)lane_id();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t key = kb0 + i * RPI + l / RC;
            const bool ok = key < a.N;
            v[i] = ok ? *reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.K) + (size_t)key * RAW +
                                                           (l % RC) * 16)
                      : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(char *base) const
    {
        const int l = (int)lane_id();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            char *dst = base + (i * RPI + l / RC) * C::ROWP;
            if constexpr (WIDEN) {
                const u32x2_t w0 = fp8x4_widen<C::MT>(v[i][0]), w1 = fp8x4_widen<C::MT>(v[i][1]);
                const u32x2_t w2 = fp8x4_widen<C::MT>(v[i][2]), w3 = fp8x4_widen<C::MT>(v[i][3]);
                *reinterpret_cast<u32x4_t *>(dst + (l % RC) * 32) = u32x4_t{w0[0], w0[1], w1[0], w1[1]};
                *reinterpret_cast<u32x4_t *>(dst + (l % RC) * 32 + 16) = u32x4_t{w2[0], w2[1], w3[0], w3[1]};
            } else {
                *reinterpret_cast<u32x4_t *>(dst + (l % RC) * 16) = v[i];
            }
        }
    }
};

// One wave alone scores keys [k_lo, k_hi) of the query whose fragments are
// in qf, 64 keys per step, and calls visit(key0, s) with lane l holding the
// (scaled) score of key key0 + l (to be masked against k_hi): with coalesced
// row loads into two register sets (two blocks in flight) and the wave's own
// LDS rows in kblk_all when they fit (WaveBlock), else with B fragments loaded
// straight from global memory (two register sets when a block's fragments
// take at most 32 registers).  The scores are bit-identical to the staged
// scan's (same MFMA order).
template <class C, class Visit>
__device__ __forceinline__ void wave_scan_range(const FusedArgs &a, const QFrags<C> &qf, char *kblk_all, int64_t k_lo,
                                                int64_t k_hi, Visit &&visit)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr bool LDSB = WaveBlock<C>::OK;
    constexpr bool PF = GlobalBlock<C>::BYTES <= 128;
    GlobalBlock<C> ga, gb;
    WaveBlock<C> wa, wbk;
    char *wl = kblk_all + (LDSB ? wave * 32 * C::ROWP : 0);
    const int boff = bfrag_lane_off<C>();
    if constexpr (LDSB) {
        wa.load(a, k_lo);
        wbk.load(a, k_lo + 32);
    } else {
        ga.load(a, k_lo);
    }
    for (int64_t key0 = k_lo; key0 < k_hi; key0 += TILE_KEYS) {
        float p0, p1;
        if constexpr (LDSB) {
            // LDS accesses of one wave complete in order, so each block's
            // fragment reads are done before the next block's rows land
            f32x16_t acc[C::HB];
            wa.store(wl);
            if (key0 + TILE_KEYS < k_hi) wa.load(a, key0 + TILE_KEYS);
            block_mfma<C>(acc, qf, wl + boff);
            p0 = reduce_block<C>(acc, qf.w);
            wbk.store(wl);
            if (key0 + TILE_KEYS + 32 < k_hi) wbk.load(a, key0 + TILE_KEYS + 32);
            block_mfma<C>(acc, qf, wl + boff);
            p1 = reduce_block<C>(acc, qf.w);
        } else if constexpr (PF) {
            gb.load(a, key0 + 32);
            p0 = ga.score(qf);
            if (key0 + TILE_KEYS < k_hi) ga.load(a, key0 + TILE_KEYS);
            p1 = gb.score(qf);
        } else {
            p0 = ga.score(qf);
            ga.load(a, key0 + 32);
            p1 = ga.score(qf);
            if (key0 + TILE_KEYS < k_hi) ga.load(a, key0 + TILE_KEYS);
        }
        float sc = combine_halves(p0, p1);
        const int64_t key = key0 + lane;
        if constexpr (C::SCALE) sc *= key < k_hi ? a.k_scale[key] : 1.f;
        visit(key0, sc);
    }
}

// ---------------------------------------------- main pass, few queries
// Few-query variant of the main scan (decoding): every wave works alone on a
// key range of one query (a.P ranges per query, a.span keys each), with the
// B fragments read straight from global K as in the recovery route, so there
// are no shared key stages and no barriers, and a single query keeps every
// SIMD of the chip busy instead of one wave per workgroup.  The scores are
// bit-identical to the staged scan's (same MFMA order); gate, binning, LDS
// histogram, refresh and compaction are those of k_fused_main, per wave.
template <class C>
__global__ __launch_bounds__(FUSED_THREADS) void k_fused_main_kp(FusedArgs a)
{
    __shared__ uint32_t whist_all[FUSED_WAVES][NBINS];
    __shared__ Cand stage_all[FUSED_WAVES][128];
    constexpr bool LDSB = WaveBlock<C>::OK;
    __shared__ __attribute__((aligned(16))) char kblk_all[LDSB ? FUSED_WAVES * 32 * C::ROWP : 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (a.force == 1) return;  // every row takes the recovery route (the sample still sets its bins)
    const int64_t gw = (int64_t)blockIdx.x * FUSED_WAVES + wave;
    const int t = (int)(gw / a.P);
    const int p = (int)(gw % a.P);
    if (t >= a.T) return;  // no barriers below: a wave may leave on its own
    const uint32_t L = kv_length(a, t);
    const int64_t k_lo = (int64_t)p * a.span;
    const int64_t k_hi = k_lo + a.span < (int64_t)L ? k_lo + a.span : (int64_t)L;
    if (k_hi <= k_lo) return;
    uint32_t *whist = whist_all[wave];
    Cand *stage = stage_all[wave];
    for (int i = lane; i < NBINS; i += 64) whist[i] = 0u;

    float off = 0.f, delta = 0.f;
    int gate_bin = 0;
    float gate_f = -__builtin_inff();
    {
        const float4 bp = a.param[t];
        const RowSample rs = row_sample(a, t, t / FUSED_WAVES, L, bp.z != 0.f);
        if (!rs.admit_all) {
            off = bp.x;
            delta = bp.y;
            const int b = wave_top_bin(a.hist + (size_t)t * NBINS, rs.q0);
            gate_bin = b > 0 ? b : 0;
            gate_f = gate_bin > 0 ? (float)gate_bin : -__builtin_inff();
        }
    }
    QFrags<C> qf;
    qf.load(a, t);
    uint32_t stage_n = 0, inrange = 0, at_gate = 0;
    Cand *cand = a.cand + (size_t)t * a.cap;
    const uint32_t cap = (uint32_t)a.cap;
    const uint32_t kq = (uint32_t)a.k;
    const bool refresh = delta > 0.f;
    auto flush = [&](uint32_t n) {
        uint32_t slot = 0;
        if (lane == 0) slot = atomicAdd(&a.tail[t], n);
        slot = lane_value(slot, 0);
        if ((uint32_t)lane < n && slot + lane < cap) cand[slot + lane] = stage[lane];
    };
    wave_scan_range<C>(a, qf, kblk_all, k_lo, k_hi, [&](int64_t key0, float s) {
        const int64_t key = key0 + lane;
        const bool valid = key < k_hi;
        const float b = fmaf(s, delta, off);
        const bool pass = valid && b >= gate_f;
        const uint64_t m = __ballot(pass);
        if (m) {
            const uint32_t bin = bin_of(b);
            const uint32_t pos = stage_n + lanes_below(m);
            if (pass) {
                atomicAdd(&whist[bin], 1u);
                stage[pos] = Cand{(uint32_t)key, s};
            }
            const uint32_t n = (uint32_t)__popcll(m);
            stage_n += n;
            inrange += n;
            at_gate += (uint32_t)__popcll(__ballot(pass && bin == (uint32_t)gate_bin));
            if (stage_n >= 64u) {
                flush(64u);
                const bool mv = (uint32_t)lane < stage_n - 64u;
                Cand e;
                if (mv) e = stage[64 + lane];
                if (mv) stage[lane] = e;
                stage_n -= 64u;
            }
            if (refresh && inrange - at_gate >= kq && gate_bin < NBINS - 1) {
                do {
                    inrange -= at_gate;
                    ++gate_bin;
                    at_gate = whist[gate_bin];
                } while (inrange - at_gate >= kq && gate_bin < NBINS - 1);
                gate_f = (float)gate_bin;
            }
        }
    });
    if (stage_n) flush(stage_n);
}


// ---------------------------------------------- recovery over the grid
// Rows whose candidates overflowed the buffer or fell short of min(k, L)
// (every row with the forced route) are recovered by the whole grid in two
// passes over their keys, the exact coarse recovery of the Sample-Guided
// Exact Top-K paper (Table 2): pass 1 builds each flagged row's full-row
// histogram over a monotone bin map, pass 2 scores the row again and
// collects every key whose bin is at or above the row's boundary bin (the
// bin of its min(k, L)-th score), which holds the exact Top-k.  The select
// kernel then selects from those candidates as for any other row; only a
// row whose boundary bin alone overflows the buffer (heavy ties, or a
// degenerate range) falls back to re-scoring inside the select kernel.
// Each flagged row is cut into key ranges, one per wave, so that a single
// recovered row occupies the whole chip.  Every workgroup lists the flagged
// rows itself, in index order, so that all agree on the work split.
constexpr int RLIST = 1024;     // flagged rows listed per round (two per thread)
constexpr int RSPAN_MIN = 512;  // keys per wave, at least

__device__ __forceinline__ bool row_needs_recovery(const FusedArgs &a, int t)
{
    const uint32_t L = kv_length(a, t);
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    if (need == 0u) return false;
    const uint32_t n = a.tail[t];
    return a.force == 1 || n > (uint32_t)a.cap || n < need;
}

// Monotone bin map of the recovery histogram: the row's sampled equal-width
// bins, or the top 11 bits of the ordered fp32 key when the sampled range
// was degenerate.
__device__ __forceinline__ uint32_t recovery_bin(float4 bp, float s)
{
    return bp.z == 0.f ? bin_of(fmaf(s, bp.y, bp.x)) : ordered_key(s) >> 21;
}

template <class C, int PASS>
__global__ __launch_bounds__(FUSED_THREADS) void k_fused_recover(FusedArgs a)
{
    static_assert(RLIST == 2 * FUSED_THREADS, "two rows per thread in the listing");
    __shared__ uint32_t list[RLIST];
    __shared__ uint32_t s_wsum[FUSED_WAVES];
    __shared__ uint32_t whist_all[PASS == 1 ? FUSED_WAVES : 1][PASS == 1 ? NBINS : 1];
    __shared__ Cand stage_all[PASS == 2 ? FUSED_WAVES : 1][128];
    constexpr bool LDSB = WaveBlock<C>::OK;
    __shared__ __attribute__((aligned(16))) char kblk_all[LDSB ? FUSED_WAVES * 32 * C::ROWP : 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t nwaves = (int64_t)gridDim.x * FUSED_WAVES;
    const int64_t gw = (int64_t)blockIdx.x * FUSED_WAVES + wave;
    for (int t0 = 0; t0 < a.T; t0 += RLIST) {
        // flagged rows of [t0, t0 + RLIST) in index order: pass 1 from the
        // candidate counts, pass 2 from the flags pass 1 set
        const int r0 = t0 + 2 * tid;
        auto flagged = [&](int t) {
            if (t >= a.T) return false;
            return PASS == 1 ? row_needs_recovery(a, t) : a.rflag[t] != 0u;
        };
        const uint32_t f0 = flagged(r0) ? 1u : 0u, f1 = flagged(r0 + 1) ? 1u : 0u;
        const uint32_t c = f0 + f1;
        const uint32_t incl = wave_incl_sum(c);
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t off = incl - c, F = 0;
#pragma unroll
        for (int w = 0; w < FUSED_WAVES; ++w) {
            if (w < wave) off += s_wsum[w];
            F += s_wsum[w];
        }
        if (f0) list[off] = (uint32_t)r0;
        if (f1) list[off + f0] = (uint32_t)(r0 + 1);
        __syncthreads();
        if (F == 0u) continue;  // workgroup-uniform
        int64_t span = ((int64_t)F * a.N + nwaves - 1) / nwaves;
        span = (span + TILE_KEYS - 1) / TILE_KEYS * TILE_KEYS;
        if (span < RSPAN_MIN) span = RSPAN_MIN;
        const int64_t per_row = (a.N + span - 1) / span;
        const int64_t items = (int64_t)F * per_row;
        for (int64_t w = gw; w < items; w += nwaves) {
            const int t = (int)list[w / per_row];
            const int64_t p = w % per_row;
            const uint32_t L = kv_length(a, t);
            const int64_t lo = p * span;
            const int64_t hi = lo + span < (int64_t)L ? lo + span : (int64_t)L;
            if (PASS == 1 && p == 0 && lane == 0) {
                a.rflag[t] = 1u;
                a.tail[t] = 0u;  // pass 2 appends from 0 (the row stays flagged: 0 < min(k, L))
            }
            if (hi <= lo) continue;
            const float4 bp = a.param[t];
            QFrags<C> qf;
            qf.load(a, t);
            if constexpr (PASS == 1) {
                uint32_t *whist = whist_all[wave];
                for (int i = lane; i < NBINS; i += 64) whist[i] = 0u;
                wave_scan_range<C>(a, qf, kblk_all, lo, hi, [&](int64_t key0, float sc) {
                    if (key0 + lane < hi) atomicAdd(&whist[recovery_bin(bp, sc)], 1u);
                });
                uint32_t *hr = a.hist_r + (size_t)t * NBINS;
                for (int i = lane; i < NBINS; i += 64) {
                    const uint32_t cnt = whist[i];
                    if (cnt) atomicAdd(&hr[i], cnt);
                }
            } else {
                const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
                const int bnd = wave_top_bin(a.hist_r + (size_t)t * NBINS, need);  // >= 0: the row holds L >= need keys
                const uint32_t B = bnd > 0 ? (uint32_t)bnd : 0u;
                Cand *stage = stage_all[wave];
                Cand *cand = a.cand + (size_t)t * a.cap;
                const uint32_t cap = (uint32_t)a.cap;
                uint32_t stage_n = 0;
                auto flush = [&](uint32_t n) {
                    uint32_t slot = 0;
                    if (lane == 0) slot = atomicAdd(&a.tail[t], n);
                    slot = lane_value(slot, 0);
                    if ((uint32_t)lane < n && slot + lane < cap) cand[slot + lane] = stage[lane];
                };
                wave_scan_range<C>(a, qf, kblk_all, lo, hi, [&](int64_t key0, float sc) {
                    const bool pass = key0 + lane < hi && recovery_bin(bp, sc) >= B;
                    const uint64_t m = __ballot(pass);
                    if (m) {
                        if (pass) stage[stage_n + lanes_below(m)] = Cand{(uint32_t)(key0 + lane), sc};
                        stage_n += (uint32_t)__popcll(m);
                        if (stage_n >= 64u) {
                            flush(64u);
                            const bool mv = (uint32_t)lane < stage_n - 64u;
                            Cand e;
                            if (mv) e = stage[64 + lane];
                            if (mv) stage[lane] = e;
                            stage_n -= 64u;
                        }
                    }
                });
                if (stage_n) flush(stage_n);
            }
        }
        __syncthreads();  // every wave is done with the list before the next round rewrites it
    }
}

// ------------------------------------------- select (+ recovery) per row
struct CandSrc {
    const Cand *c;
    uint32_t n;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
            const Cand e = c[i];
            f(e.idx, e.val);
        }
    }
};

// Re-scores every valid key of row t (each wave takes every 4th tile, with
// B fragments read straight from global memory).
template <class C>
struct RescoreSrc {
    const FusedArgs *a;
    int t;
    uint32_t L;
    template <class F>
    __device__ void for_each(F &&f) const
    {
        const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
        const int lane = (int)lane_id();
        QFrags<C> qf;
        qf.load(*a, t);
        for (int64_t key0 = (int64_t)wave * TILE_KEYS; key0 < (int64_t)L; key0 += (int64_t)nw * TILE_KEYS) {
            float s = tile_scores_global<C>(qf, *a, key0);
            const int64_t key = key0 + lane;
            if (key < (int64_t)L) {
                if constexpr (C::SCALE) s *= a->k_scale[key];
                f((uint32_t)key, s);
            }
        }
    }
};

enum { FROUTE_SAMPLE = 1, FROUTE_RECOVER = 3, FROUTE_ALL = 4, FROUTE_GRID_RECOVERY = 5 };

// After the grid-wide recovery passes every row holds at least min(k, L)
// candidates; a row whose candidates still overflow the buffer (its boundary
// bin alone holds more keys than the buffer) is re-scored from Q and K by
// k_fused_rescore instead of being selected from the buffer.
__device__ __forceinline__ bool select_rescores(const FusedArgs &a, int t, uint32_t need)
{
    const uint32_t n = a.tail[t];
    return n > (uint32_t)a.cap || n < need;
}

template <class C>
__global__ __launch_bounds__(SEL_THREADS_HR) void k_fused_select(FusedArgs a)
{
    __shared__ SelectSmem sm;
    const int tid = threadIdx.x;
    const int t = blockIdx.x;
    const uint32_t L = kv_length(a, t);
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    int32_t *oi = a.out_idx + (size_t)t * a.k;
    float *os = a.out_score + (size_t)t * a.k;
    for (uint32_t i = need + tid; i < (uint32_t)a.k; i += SEL_THREADS_HR) {
        oi[i] = -1;
        os[i] = -__builtin_inff();
    }
    if (need == 0) {
        if (tid == 0 && a.route) a.route[t] = FROUTE_ALL;
        if (tid == 0 && a.count) a.count[t] = 0;
        return;
    }
    const uint32_t n = a.tail[t];
    const bool recover = select_rescores(a, t, need);  // left to k_fused_rescore
    auto emit = [&](uint32_t slot, uint64_t K) {
        if (slot < need) {
            oi[slot] = (int32_t)key_index(K);
            os[slot] = key_value(K);
        }
    };
    if (!recover) {
        CandSrc src{a.cand + (size_t)t * a.cap, n};
        if (n <= (uint32_t)STASH_CAP) {
            // all candidates fit on chip: one parallel copy, then every
            // refinement round reads LDS only
            constexpr int B = 8;  // loads in flight per thread
            float mn = __builtin_inff(), mx = -__builtin_inff();  // value range, taken on the way
            for (uint32_t i0 = 0; i0 < n; i0 += SEL_THREADS_HR * B) {
                Cand e[B];
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    const uint32_t i = i0 + j * SEL_THREADS_HR + tid;
                    if (i < n) e[j] = src.c[i];
                }
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    const uint32_t i = i0 + j * SEL_THREADS_HR + tid;
                    if (i < n) {
                        sm.stash[i] = make_key(e[j].val, e[j].idx);
                        mn = fminf(mn, e[j].val);
                        mx = fmaxf(mx, e[j].val);
                    }
                }
            }
            mn = wave_min(mn);
            mx = wave_max(mx);
            if ((tid & 63) == 0) {
                sm.vmin[tid >> 6] = mn;
                sm.vmax[tid >> 6] = mx;
            }
            __syncthreads();
            select_stashed<SEL_THREADS_HR>(sm, n, need, emit, true);
        } else {
            exact_select<SEL_THREADS_HR>(sm, src, need, emit);
        }
    }
    if (tid == 0 && a.count) a.count[t] = (int32_t)n;
    if (tid == 0 && a.route) {
        const float4 bp = a.param[t];
        const RowSample rs = row_sample(a, t, t / FUSED_WAVES, L, bp.z != 0.f);
        a.route[t] = recover ? FROUTE_RECOVER
                             : (a.rflag[t] ? FROUTE_GRID_RECOVERY : (rs.admit_all ? FROUTE_ALL : FROUTE_SAMPLE));
    }
}

// Re-scores row t from Q and K and selects it exactly (one workgroup).
template <class C>
__device__ void rescore_row(const FusedArgs &a, int t, SelectSmem &sm)
{
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
    RescoreSrc<C> src{&a, t, L};
    exact_select<SEL_THREADS_HR>(sm, src, need, emit);
    __syncthreads();  // the next row reuses sm
}

__device__ __forceinline__ bool row_rescores(const FusedArgs &a, int t)
{
    const uint32_t L = kv_length(a, t);
    const uint32_t need = L < (uint32_t)a.k ? L : (uint32_t)a.k;
    return need != 0 && select_rescores(a, t, need);
}

// The re-scoring route of the selection, for the rows select_rescores
// names: every valid key of the row is re-scored from Q and K (RescoreSrc,
// the scan's MFMA order, so the scores equal the scan's) and the row is
// selected exactly by one workgroup.  A kernel of its own, so that the
// selection does not carry the re-scoring registers (Q fragments and
// accumulators) on every row.  Such rows are rare: RESCORE_GROUPS workgroups
// share the rows (workgroup b takes rows b, b + gridDim.x, ...), and each
// checks its rows a chunk of one row per thread at a time, with one vote, so
// that a call with nothing to re-score costs about one memory round trip.
template <class C>
__global__ __launch_bounds__(SEL_THREADS_HR) void k_fused_rescore(FusedArgs a)
{
    __shared__ SelectSmem sm;
    for (int base = 0; blockIdx.x + (int64_t)base * gridDim.x < a.T; base += SEL_THREADS_HR) {
        const int64_t ti = blockIdx.x + (int64_t)(base + threadIdx.x) * gridDim.x;
        if (!__syncthreads_or(ti < a.T && row_rescores(a, (int)ti))) continue;
        for (int j = 0; j < SEL_THREADS_HR; ++j) {
            const int64_t tj = blockIdx.x + (int64_t)(base + j) * gridDim.x;
            if (tj >= a.T) break;
            const int t = (int)tj;
            if (!row_rescores(a, t)) continue;  // workgroup-uniform
            rescore_row<C>(a, t, sm);
        }
    }
}

// --------------------------------------------------------------- launch
template <class C>
hipError_t launch_fused_cfg(const FusedPlan &p, const FusedArgs &a, hipStream_t stream)
{
    hipError_t e;
    {
        StageTimer st(ST_F_MINMAX, stream);
        e = hipSuccess;
        if (a.pidx) {
            const int64_t threads = p.np * (a.rowb / 16);
            e = launch_kernel(k_prior_gather<C>, dim3((unsigned)((threads + 255) / 256)), dim3(256), stream, a);
        }
        if (e == hipSuccess)
            e = a.pidx ? launch_kernel(k_fused_minmax<C, true>, dim3(p.G * p.Ps), dim3(FUSED_THREADS), stream, a)
                       : launch_kernel(k_fused_minmax<C, false>, dim3(p.G * p.Ps), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_HIST, stream);
        e = a.samp ? launch_kernel(k_fused_samplehist<C, true>, dim3(p.G * p.Ps), dim3(FUSED_THREADS), stream, a)
                   : launch_kernel(k_fused_samplehist<C, false>, dim3(p.G * p.Ps), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_MAIN, stream);
        if (p.kp)
            e = launch_kernel(k_fused_main_kp<C>, dim3((unsigned)((int64_t)p.T * p.P / FUSED_WAVES)),
                              dim3(FUSED_THREADS), stream, a);
        else
            e = launch_kernel(k_fused_main<C>, dim3(p.G * p.P), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_RECOVER, stream);
        e = launch_kernel(k_fused_recover<C, 1>, dim3(RECOVER_WGS), dim3(FUSED_THREADS), stream, a);
        if (e == hipSuccess) e = launch_kernel(k_fused_recover<C, 2>, dim3(RECOVER_WGS), dim3(FUSED_THREADS), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_SELECT, stream);
        e = launch_kernel(k_fused_select<C>, dim3(p.T), dim3(SEL_THREADS_HR), stream, a);
    }
    if (e != hipSuccess) return e;
    {
        StageTimer st(ST_F_RESCORE, stream);
        e = launch_kernel(k_fused_rescore<C>, dim3(p.T < RESCORE_GROUPS ? p.T : RESCORE_GROUPS), dim3(SEL_THREADS_HR),
                          stream, a);
    }
    return e;
}

using FusedLauncher = hipError_t (*)(const FusedPlan &, const FusedArgs &, hipStream_t);

// Registry of instantiated configurations (filled by the per-dtype units).
FusedLauncher find_fused_launcher(int qt, int kt, int hb, int d, bool relu, bool q8);

#define ITK_FUSED_CASES_FOR(QT, KT)                                                               \
    if (qt == QT && kt == KT) {                                                                   \
        if (relu) {                                                                               \
            if (hb == 1 && d == 64) return &launch_fused_cfg<FCfg<QT, KT, 1, 64, true>>;          \
            if (hb == 1 && d == 128) return &launch_fused_cfg<FCfg<QT, KT, 1, 128, true>>;        \
            if (hb == 1 && d == 256) return &launch_fused_cfg<FCfg<QT, KT, 1, 256, true>>;        \
            if (hb == 2 && d == 64) return &launch_fused_cfg<FCfg<QT, KT, 2, 64, true>>;          \
            if (hb == 2 && d == 128) return &launch_fused_cfg<FCfg<QT, KT, 2, 128, true>>;        \
        } else {                                                                                  \
            if (hb == 1 && d == 64) return &launch_fused_cfg<FCfg<QT, KT, 1, 64, false>>;         \
            if (hb == 1 && d == 128) return &launch_fused_cfg<FCfg<QT, KT, 1, 128, false>>;       \
            if (hb == 1 && d == 256) return &launch_fused_cfg<FCfg<QT, KT, 1, 256, false>>;       \
        }                                                                                         \
    }

// FP8 scoring (queries quantized per row, FP8 keys copied raw).
#define ITK_FUSED_Q8_CASES_FOR(QT)                                                                \
    if (qt == QT && kt == ITK_FP8_E4M3 && q8) {                                                   \
        if (relu) {                                                                               \
            if (hb == 1 && d == 64) return &launch_fused_cfg<FCfg<QT, ITK_FP8_E4M3, 1, 64, true, true>>;   \
            if (hb == 1 && d == 128) return &launch_fused_cfg<FCfg<QT, ITK_FP8_E4M3, 1, 128, true, true>>; \
            if (hb == 1 && d == 256) return &launch_fused_cfg<FCfg<QT, ITK_FP8_E4M3, 1, 256, true, true>>; \
            if (hb == 2 && d == 64) return &launch_fused_cfg<FCfg<QT, ITK_FP8_E4M3, 2, 64, true, true>>;   \
            if (hb == 2 && d == 128) return &launch_fused_cfg<FCfg<QT, ITK_FP8_E4M3, 2, 128, true, true>>; \
        }                                                                                         \
        return nullptr;                                                                           \
    }

// fp32 operands: ceil(H/32) * D <= 128 keeps the Q fragments within budget.
#define ITK_FUSED_CASES_F32                                                                       \
    if (qt == ITK_F32 && kt == ITK_F32) {                                                         \
        if (hb == 1 && d == 64) return relu ? &launch_fused_cfg<FCfg<ITK_F32, ITK_F32, 1, 64, true>>        \
                                            : &launch_fused_cfg<FCfg<ITK_F32, ITK_F32, 1, 64, false>>;      \
        if (hb == 1 && d == 128) return relu ? &launch_fused_cfg<FCfg<ITK_F32, ITK_F32, 1, 128, true>>      \
                                             : &launch_fused_cfg<FCfg<ITK_F32, ITK_F32, 1, 128, false>>;    \
        if (hb == 2 && d == 64 && relu) return &launch_fused_cfg<FCfg<ITK_F32, ITK_F32, 2, 64, true>>;    \
    }

}  // namespace itk
