/* Attainable-peak probes for MI355X (gfx950): the reference kernels that the
 * measurements of the DSA hot path are compared against besides the vendor
 * peaks.  They are not part of the hot path and compute nothing of the
 * method; bench.py times them with events on the stream it passes.
 *
 * Built as libdsa_probes.so next to libdsa.so.  Both calls only enqueue work
 * on `stream` (a hipStream_t, NULL = the default stream); they never
 * allocate, copy to the host or synchronise.  They return 0 on success or the
 * hipError_t value of a failed launch, and -1 for invalid arguments (checked
 * before any launch, so an invalid call has no device side effects).
 */
#ifndef DSA_PROBES_H
#define DSA_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory `buf` once, in 2 KiB tiles moved by
 * global_load_lds_dwordx4 with the streaming hint into a per-wave LDS ring
 * (the load path of the decode indexer), and writes one word per thread of
 * the grid into `sink` so that the reads cannot be elided.
 *   buf        device pointer, 16-byte aligned; bytes: a positive multiple of 2048
 *   sink       device pointer to sink_words 32-bit words; needs at least
 *              dsa_probe_stream_read_sink_words(bytes) of them
 * The data read is arbitrary; the sink values carry no meaning. */
int dsa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream);
int64_t dsa_probe_stream_read_sink_words(int64_t bytes);

/* Keeps every SIMD issuing independent bf16 matrix-core instructions for
 * `iters` iterations, with no memory traffic in the loop: form 0 =
 * v_mfma_f32_16x16x32_bf16 (8 accumulator chains per wave), form 1 =
 * v_mfma_f32_32x32x16_bf16 (4 chains per wave).  One float per thread goes
 * to `sink` (at least dsa_probe_mfma_sink_words() of them).
 * dsa_probe_mfma_flops(form, iters) is the work one launch does (2 flops per
 * multiply-add), for the rate; it returns -1 for an unknown form. */
int dsa_probe_mfma(int form, int iters, float* sink, int64_t sink_words, void* stream);
int64_t dsa_probe_mfma_sink_words(void);
double dsa_probe_mfma_flops(int form, int iters);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PROBES_H */
