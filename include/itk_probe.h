/* Test-only probes of the device building blocks of the Indexer-TopK
 * library.  They live in a library of their own, libitk_probe.so, which the
 * tests (MFMA lane layout and accumulation, FP8 widening, the coarse key) and
 * the benchmark's streaming-read ceiling load; the product library
 * libitk.so exports none of them.  Same conventions as itk.h: device
 * pointers, `stream` a hipStream_t (NULL: the default stream), asynchronous
 * launches, ITK_ERR_INVALID_ARG for bad arguments, ITK_ERR_HIP when a launch
 * fails. */
#ifndef ITK_PROBE_H
#define ITK_PROBE_H

#include "itk.h"

#ifdef __cplusplus
extern "C" {
#endif

/*  itk_debug_mfma: one 32x32 MFMA (mtype 0 bf16 x16, 1 fp16 x16, 2 fp32 x2,
 *    3 e4m3fn x64 with unit block scales, 4 the same onto the accumulator
 *    values that c_out holds on entry);
 *    lane l reads its A and B operand fragments from a_frags[l], b_frags[l]
 *    (16 bytes each for bf16/fp16, 4 bytes for fp32, 32 for e4m3fn) and writes its 16
 *    accumulator values to c_out[16 l .. 16 l + 15].
 *  itk_debug_fp8: widen n e4m3fn codes to bf16 and fp16 bit patterns.
 *  itk_debug_coarse: the 11-bit coarse key of x[i] and the inclusive fp32
 *    endpoint of coarse bin i, for i < n <= 2048.
 *  itk_debug_stream_read: reads floor(bytes / 16) 16-byte chunks of x (16-byte
 *    aligned) with the non-temporal loads of the ragged scan over `blocks`
 *    workgroups of 256 threads and writes each workgroup's maximum to
 *    out[blocks]: the HBM read rate a plain streaming read reaches. */
itk_status itk_debug_mfma(int32_t mtype, const void *a_frags, const void *b_frags, float *c_out, void *stream);
itk_status itk_debug_fp8(const uint8_t *in, uint16_t *bf16_out, uint16_t *f16_out, int32_t n, void *stream);
itk_status itk_debug_coarse(const float *x, uint32_t *key_out, float *endpoint_out, int32_t n, void *stream);
itk_status itk_debug_stream_read(const void *x, uint64_t bytes, float *out, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ITK_PROBE_H */
