/*
 * Ceiling probes of the compressed sparse attention library: the attainable HBM read bandwidth
 * (streamed and gathered by row) and matrix-core rate of the part the library runs on, measured with the same kind of instructions its
 * kernels use, so that a kernel's roofline fraction can be stated against a measured ceiling beside
 * the vendor's figure. They compute nothing of the layer.
 *
 * All calls are asynchronous on `stream` (a hipStream_t, NULL = the default stream) and return
 * CSA_OK (0) or CSA_ERR_ARG (-1) / CSA_ERR_HIP (-4), with the message in csa_last_error().
 */
#ifndef CSA_PROBE_H
#define CSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` of device memory at `buf` (16-byte aligned, bytes a multiple of 16) once with 16-byte
 * vector loads, grid-stride over every compute unit, and writes one 32-bit word per thread of the
 * launch into `sink` (device, at least csa_probe_sink_words() words) so that no load is dead.
 */
int csa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Reads n_rows rows of `row_bytes` bytes each (a multiple of 16, at most 1 MiB) gathered from `buf`
 * (device, 16-byte aligned, `buf_bytes` long): row r is buf + idx[r] * row_bytes, idx a device int32
 * array [n_rows] (row numbers outside [0, buf_bytes / row_bytes) are clamped into it). One wave per
 * row with four rows in flight per wave, 16-byte loads; writes one 32-bit word per thread of the
 * launch into `sink` (at least csa_probe_sink_words() words). This is the access pattern of the sparse
 * attention's gathered entries, so its counters calibrate the attention's.
 */
int csa_probe_gather_read(const void* buf, size_t buf_bytes, size_t row_bytes, const int32_t* idx, int64_t n_rows,
                          uint32_t* sink, void* stream);

/*
 * Runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 chains in every wave of a grid
 * of csa_probe_sink_words() / 64 waves (eight per compute unit), 4 * 32768 * iters FLOP per wave;
 * each wave writes its accumulators' sum to sink[wave]. iters >= 1.
 */
int csa_probe_mfma_bf16(int iters, float* sink, void* stream);

/* Words of `sink` both probes need (one per thread of their launch). */
size_t csa_probe_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_PROBE_H */
