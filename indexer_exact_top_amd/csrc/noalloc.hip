// topk_ragged_noalloc: the standalone ragged Top-k with its scratch in a
// static device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// `scratch` below is a host-side stand-in for the device array: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever passed to kernels.  Every
// call on a GPU shares that GPU's array, so calls that overlap on one GPU
// race; the ragged kernels write every scratch word they later read within
// the same call, so nothing needs clearing between calls.
#include <mutex>

#include "itk_internal.hpp"

namespace itk {
namespace {

static __device__ __align__(256) unsigned char scratch[ITK_RAGGED_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// Device address of `scratch` on the current device (looked up on first use).
hipError_t scratch_on_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace itk

extern "C" itk_status topk_ragged_noalloc(const float *scores, int64_t row_pitch, const int32_t *row_len, int32_t M,
                                          int32_t k, int32_t *out_idx, void *stream)
{
    using namespace itk;
    itk_status st;
    if (ragged_trivial(M, row_pitch, k, out_idx, static_cast<hipStream_t>(stream), &st)) return st;
    if (!scores || !row_len || !out_idx) return ITK_ERR_INVALID_ARG;
    if (row_pitch > (int64_t)0x7FFFFFFF) return ITK_ERR_UNSUPPORTED;
    const RaggedPlan p = plan_ragged(M, row_pitch, k);
    if (p.bytes > (size_t)ITK_RAGGED_NOALLOC_SCRATCH_BYTES) return ITK_ERR_SCRATCH_LIMIT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ITK_ERR_HIP;
    if (s) {  // the scratch used is the current device's: the stream must be on it
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return ITK_ERR_HIP;
        if (sdev != cur) return ITK_ERR_INVALID_ARG;
    }
    void *ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess) return ITK_ERR_HIP;
    return launch_ragged(p, scores, row_len, out_idx, ws, s) == hipSuccess ? ITK_OK : ITK_ERR_HIP;
}
