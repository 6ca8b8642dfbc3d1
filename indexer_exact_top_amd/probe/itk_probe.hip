// Test-only probes of the layouts and conversions the fused kernels rely on,
// built into their own library (libitk_probe.so, declared in itk_probe.h) so
// that the product library carries none of them.  They compile the product's
// device building blocks from the same headers.
#include "fused_impl.hpp"
#include "itk_probe.h"

namespace itk {

// One 32x32 MFMA: lane l loads its A and B fragments from a[l], b[l] and
// stores its 16 accumulator values to c[l*16 .. l*16+15].
template <int MT>
__global__ void k_debug_mfma(const typename MTraits<MT>::frag *a, const typename MTraits<MT>::frag *b, float *c)
{
    const int l = threadIdx.x;
    f32x16_t acc = f32x16_t{};
    acc = mfma32<MT>(a[l], b[l], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// The FP8 MFMA with an accumulator input: lane l's 16 accumulator values
// start from c[l*16 .. l*16+15] (the chained k-steps of the FP8 scan add
// onto the previous step's sums).
__global__ void k_debug_mfma_fp8_acc(const u32x8_t *a, const u32x8_t *b, float *c)
{
    const int l = threadIdx.x;
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = c[l * 16 + r];
    acc = mfma32<M_FP8>(a[l], b[l], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// Widens codes 4 at a time, as the key staging does (a partial last group
// is padded with zero codes, which are not stored).
__global__ void k_debug_fp8(const uint8_t *in, uint16_t *bf, uint16_t *hf, int n)
{
    const int i0 = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (i0 >= n) return;
    uint32_t word = 0;
    for (int j = 0; j < 4 && i0 + j < n; ++j) word |= (uint32_t)in[i0 + j] << (8 * j);
    const u32x2_t b = fp8x4_widen<M_BF16>(word), h = fp8x4_widen<M_F16>(word);
    for (int j = 0; j < 4 && i0 + j < n; ++j) {
        bf[i0 + j] = (uint16_t)(b[j >> 1] >> (16 * (j & 1)));
        hf[i0 + j] = (uint16_t)(h[j >> 1] >> (16 * (j & 1)));
    }
}

__global__ void k_debug_coarse(const float *x, uint32_t *key, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) key[i] = coarse_key(x[i]);
}

// One wave per bin: the endpoint exactly as the standalone scan computes it.
__global__ void k_debug_endpoint(float *endpoint)
{
    const float e = coarse_endpoint_wave(blockIdx.x);
    if (threadIdx.x == 0) endpoint[blockIdx.x] = e;
}

}  // namespace itk

using namespace itk;

// Streaming read of n16 16-byte chunks with the loads of the ragged scan
// (non-temporal, eight in flight per thread): a max-reduction whose only
// output is one word per workgroup, so the kernel's time is the read.
__global__ __launch_bounds__(256) void k_debug_stream_read(const f32x4_t *x, uint64_t n16, float *out)
{
    constexpr int U = 8;
    const uint64_t stride = (uint64_t)gridDim.x * 256u;
    float m = -__builtin_inff();
    for (uint64_t base = (uint64_t)blockIdx.x * 256u + threadIdx.x; base < n16; base += stride * U) {
        f32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * stride;
            v[u] = i < n16 ? __builtin_nontemporal_load(x + i) : f32x4_t{m, m, m, m};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) m = fmaxf(m, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    }
    m = wave_max(m);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

extern "C" {

itk_status itk_debug_mfma(int32_t mtype, const void *a_frags, const void *b_frags, float *c_out, void *stream)
{
    if (!a_frags || !b_frags || !c_out) return ITK_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mtype == M_BF16)
        e = launch_kernel(k_debug_mfma<M_BF16>, dim3(1), dim3(64), s, static_cast<const u32x4_t *>(a_frags),
                          static_cast<const u32x4_t *>(b_frags), c_out);
    else if (mtype == M_F16)
        e = launch_kernel(k_debug_mfma<M_F16>, dim3(1), dim3(64), s, static_cast<const u32x4_t *>(a_frags),
                          static_cast<const u32x4_t *>(b_frags), c_out);
    else if (mtype == M_F32)
        e = launch_kernel(k_debug_mfma<M_F32>, dim3(1), dim3(64), s, static_cast<const float *>(a_frags),
                          static_cast<const float *>(b_frags), c_out);
    else if (mtype == M_FP8)
        e = launch_kernel(k_debug_mfma<M_FP8>, dim3(1), dim3(64), s, static_cast<const u32x8_t *>(a_frags),
                          static_cast<const u32x8_t *>(b_frags), c_out);
    else if (mtype == M_FP8 + 1)
        e = launch_kernel(k_debug_mfma_fp8_acc, dim3(1), dim3(64), s, static_cast<const u32x8_t *>(a_frags),
                          static_cast<const u32x8_t *>(b_frags), c_out);
    else
        return ITK_ERR_INVALID_ARG;
    return e == hipSuccess ? ITK_OK : ITK_ERR_HIP;
}

itk_status itk_debug_fp8(const uint8_t *in, uint16_t *bf16_out, uint16_t *f16_out, int32_t n, void *stream)
{
    if (!in || !bf16_out || !f16_out || n <= 0) return ITK_ERR_INVALID_ARG;
    const hipError_t e = launch_kernel(k_debug_fp8, dim3((n + 1023) / 1024), dim3(256),
                                       static_cast<hipStream_t>(stream), in, bf16_out, f16_out, n);
    return e == hipSuccess ? ITK_OK : ITK_ERR_HIP;
}

itk_status itk_debug_coarse(const float *x, uint32_t *key_out, float *endpoint_out, int32_t n, void *stream)
{
    if (!x || !key_out || !endpoint_out || n <= 0 || n > NBINS) return ITK_ERR_INVALID_ARG;
    if (launch_kernel(k_debug_coarse, dim3((n + 255) / 256), dim3(256), static_cast<hipStream_t>(stream), x, key_out,
                      n) != hipSuccess)
        return ITK_ERR_HIP;
    return launch_kernel(k_debug_endpoint, dim3(n), dim3(64), static_cast<hipStream_t>(stream), endpoint_out) ==
                   hipSuccess
               ? ITK_OK
               : ITK_ERR_HIP;
}

itk_status itk_debug_stream_read(const void *x, uint64_t bytes, float *out, int32_t blocks, void *stream)
{
    if (!x || !out || bytes < 16 || blocks <= 0 || (reinterpret_cast<uintptr_t>(x) & 15u)) return ITK_ERR_INVALID_ARG;
    return launch_kernel(k_debug_stream_read, dim3(blocks), dim3(256), static_cast<hipStream_t>(stream),
                         static_cast<const f32x4_t *>(x), (uint64_t)(bytes / 16), out) == hipSuccess
               ? ITK_OK
               : ITK_ERR_HIP;
}

}  // extern "C"
