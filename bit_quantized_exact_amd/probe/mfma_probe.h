/*
 * mfma_probe.h - measurement helpers of libattn_probe.so, a small library
 * of its own beside libattn.so.  They are not part of the attention path and
 * not part of its C ABI: the benchmark uses them to report the sustained
 * matrix-core rate and the streaming read bandwidth of the device next to the
 * published peaks, so that a kernel's fraction of a peak can be read against
 * what a dense MFMA loop or a plain read reaches on the same part.
 */
#ifndef ATTN_MFMA_PROBE_H
#define ATTN_MFMA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Dense MFMA loop.  kind 0: v_mfma_f32_32x32x16_f16, kind 1:
 * v_mfma_i32_32x32x32_i8; kind 2: the FP16 loop with softmax-like vector work
 * beside each MFMA (one exp2 and five FMAs on independent registers), kind 3:
 * that vector work alone.  Launches `blocks` workgroups of 256 threads (two
 * per compute unit give two waves per SIMD) on `stream` (a hipStream_t, NULL
 * = null stream); each wave runs `iters` rounds of 4 independent chains and
 * writes one fp32 value per thread to `sink` (DEVICE memory, blocks * 256
 * floats, owned by the caller).  *ops (HOST, may be NULL) receives the MFMA
 * operations one launch of kind 0, 1 or 2 performs (2 * 32 * 32 * K per MFMA;
 * kind 3 reports kind 2's count).  Returns 0, -1 for a bad argument (nothing
 * launched), -3 when the launch failed. */
int attn_probe_mfma(int kind, int blocks, int iters, float* sink, double* ops, void* stream);

/* Streaming read of `bytes` bytes of DEVICE memory at `buf` (16-byte
 * aligned, bytes a multiple of 16, owned by the caller): `blocks` workgroups
 * of 256 threads read it once in 16-byte non-temporal loads, four in flight
 * per thread, and each thread writes the XOR of what it read, as a float, to `sink`
 * (DEVICE memory, blocks * 256 floats).  The practical read bandwidth of the
 * part, reported beside the 8 TB/s published peak for the HBM-bound kernels
 * (decode, quantisation).  Returns 0, -1 for a bad argument (nothing
 * launched), -3 when the launch failed. */
int attn_probe_hbm_read(const void* buf, unsigned long long bytes, int blocks, float* sink, void* stream);

/* Compute units of the current device into *cus (HOST).  Returns 0, -1 for a
 * NULL pointer or no device, -3 when the query failed. */
int attn_probe_compute_units(int* cus);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MFMA_PROBE_H */
