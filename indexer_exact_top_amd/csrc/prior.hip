// History sample for the fused Indexer-TopK (LiteTopK, Sec. 3.2 "Sampling"):
// the k' keys that occur most often in the previous chunk's Top-k lists.
//
// Prefix keys are shared across the chunks of a prefill, and adjacent chunks
// tend to attend to the same prefix tokens, so these keys are likely to score
// high again; scored first, they give the next chunk a tight initial gate.
//
// Three small kernels count the occurrences of every key in [0, N) into an
// fp32 row (a count is a small integer, exact in fp32 while the lists hold at
// most 2^24 entries), and the exact ragged Top-k of that single row takes the
// k' largest counts, equal counts in favour of the lower index.
#include "itk_internal.hpp"
#include "itk_device.hpp"

namespace itk {

namespace {

constexpr int PR_THREADS = 256;
typedef uint32_t pr_u32x4 __attribute__((ext_vector_type(4)));

// Zeroes the count row (16 bytes per thread) and stores its valid length.
__global__ __launch_bounds__(PR_THREADS) void k_prior_clear(uint32_t *cnt, int64_t words4, int32_t *row_len, int32_t N)
{
    const int64_t i = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
    if (i < words4) reinterpret_cast<pr_u32x4 *>(cnt)[i] = pr_u32x4{0u, 0u, 0u, 0u};
    if (i == 0) row_len[0] = N;
}

// One atomic increment per list entry that names a key in [0, N).
__global__ __launch_bounds__(PR_THREADS) void k_prior_count(const int32_t *prev, int64_t n, uint32_t *cnt, int64_t N)
{
    const int64_t stride = (int64_t)gridDim.x * PR_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x; i < n; i += stride) {
        const int32_t j = prev[i];
        if (j >= 0 && (int64_t)j < N) atomicAdd(&cnt[j], 1u);
    }
}

// Counts -> fp32 in place (exact: every count is at most 2^24).
__global__ __launch_bounds__(PR_THREADS) void k_prior_to_float(uint32_t *cnt, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
    if (i < N) reinterpret_cast<float *>(cnt)[i] = (float)cnt[i];
}

}  // namespace

itk_status plan_prior(int32_t T_prev, int32_t k, int64_t N, int32_t k_prime, PriorPlan *out)
{
    if (T_prev < 0 || k <= 0 || N <= 0 || k_prime <= 0) return ITK_ERR_INVALID_ARG;
    if (N > (int64_t)0x7FFFFFFF) return ITK_ERR_UNSUPPORTED;
    if ((int64_t)T_prev * k > ((int64_t)1 << 24)) return ITK_ERR_UNSUPPORTED;  // counts exact in fp32
    PriorPlan p;
    p.N = N; p.T_prev = T_prev; p.k = k; p.k_prime = k_prime;
    const int64_t pitch = (N + 3) / 4 * 4;
    p.rag = plan_ragged(1, pitch, k_prime);
    size_t off = 0;
    p.off_count = off; off = align256(off + (size_t)pitch * sizeof(uint32_t) + 256);  // row, then its length
    p.off_rag = off; off = align256(off + p.rag.bytes);
    p.bytes = off;
    *out = p;
    return ITK_OK;
}

hipError_t launch_prior(const PriorPlan &p, const int32_t *prev_idx, int32_t *prior_out, void *ws, hipStream_t stream)
{
    char *w = static_cast<char *>(ws);
    const int64_t pitch = p.rag.pitch;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(w + p.off_count);
    int32_t *row_len = reinterpret_cast<int32_t *>(w + p.off_count + align256((size_t)pitch * sizeof(uint32_t)));
    const int64_t words4 = pitch / 4;
    hipError_t e = launch_kernel(k_prior_clear, dim3((unsigned)((words4 + PR_THREADS - 1) / PR_THREADS)),
                                 dim3(PR_THREADS), stream, cnt, words4, row_len, (int32_t)p.N);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)p.T_prev * p.k;
    if (n > 0) {
        int64_t blocks = (n + PR_THREADS - 1) / PR_THREADS;
        if (blocks > 4096) blocks = 4096;
        e = launch_kernel(k_prior_count, dim3((unsigned)blocks), dim3(PR_THREADS), stream, prev_idx, n, cnt, p.N);
        if (e != hipSuccess) return e;
    }
    e = launch_kernel(k_prior_to_float, dim3((unsigned)((p.N + PR_THREADS - 1) / PR_THREADS)), dim3(PR_THREADS),
                      stream, cnt, p.N);
    if (e != hipSuccess) return e;
    return launch_ragged(p.rag, reinterpret_cast<const float *>(cnt), row_len, prior_out, w + p.off_rag, stream);
}

}  // namespace itk
