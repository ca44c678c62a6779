/*
 * sckv_peak.h -- measurement kernels for the roofline denominators of the
 * compressed sparse attention library (libsckv_peak.so, gfx950).
 *
 * Not part of the hot path: these calls re-measure, on the GPU at hand, the
 * quantities the hot path's kernels are judged against -- streaming HBM
 * bandwidth (a copy and a read-only pass over buffers far larger than the
 * last-level cache), the rate of 1 KiB row gathers (the attention's access
 * pattern) and the dense matrix-core rate for the two contractions the
 * library runs (bf16 products, and e2m1 x e2m1 products with power-of-two block
 * scales).  The caller times them (e.g. with HIP events on `stream`).
 *
 * Conventions as in sckv.h: device pointers, a hipStream_t as void*, calls only
 * enqueue work, host checks first, 0 or a negative sckv_status (declared in
 * sckv.h) with sckv_peak_last_error() describing a failure.
 */
#ifndef SCKV_PEAK_H_
#define SCKV_PEAK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sckv_peak_copy -- dst[0 .. bytes) = src[0 .. bytes) with 16-byte streaming
 * (non-temporal) vector loads and stores, `blocks` workgroups of 256 threads
 * striding over the buffer, each thread keeping `depth` (4, 8 or 16) loads in
 * flight.  bytes must be a multiple of 64 and both pointers 16-byte aligned;
 * the buffers must not overlap.  Moves 2 * bytes through HBM.
 */
int sckv_peak_copy(const void* src, void* dst, int64_t bytes, int blocks, int depth, void* stream);

/*
 * sckv_peak_read -- reads src[0 .. bytes) once (16-byte streaming vector
 * loads, `depth` in flight a thread, XOR folded per thread) and writes one
 * 32-bit word per thread to out [blocks * 256], so the loads cannot be
 * dropped.  bytes a multiple of 64, src 16-byte aligned.
 */
int sckv_peak_read(const void* src, int64_t bytes, uint32_t* out, int blocks, int depth, void* stream);

/*
 * sckv_peak_gather -- reads the 1 KiB rows rows[idx[i]] for i in [0, n_idx)
 * (rows [n_rows][1024 bytes], 16-byte aligned; every idx[i] in [0, n_rows),
 * which the caller guarantees: it is not checked on the device) with one
 * 16-byte load a lane per row, each wave keeping `depth` (4, 8 or 16) rows in
 * flight, `blocks` workgroups of 256 threads striding over the list; XOR
 * folded per thread into out [blocks * 256].  Moves n_idx KiB from HBM when
 * the rows are spread over far more than the last-level cache.
 */
int sckv_peak_gather(const void* rows, int64_t n_rows, const int32_t* idx, int64_t n_idx, uint32_t* out, int blocks,
                     int depth, void* stream);

/* Matrix-core loop kinds. */
enum sckv_peak_mfma_kind {
    SCKV_PEAK_MFMA_BF16 = 0, /* v_mfma_f32_32x32x16_bf16: 32768 flops an instruction */
    SCKV_PEAK_MFMA_FP4 = 1   /* v_mfma_scale_f32_32x32x64_f8f6f4, e2m1 x e2m1: 131072 flops */
};

/*
 * sckv_peak_mfma -- `blocks` workgroups of 256 threads (4 waves); every wave
 * runs `iters` rounds of 8 independent matrix-core products of `kind` on
 * register operands, then writes one float per thread to out [blocks * 256].
 * The flops of the launch are sckv_peak_mfma_flops(kind, iters, blocks).
 */
int sckv_peak_mfma(int kind, int64_t iters, int blocks, float* out, void* stream);

/* Floating-point operations (multiply and add counted separately) of one
 * sckv_peak_mfma launch; 0 for an unknown kind. */
double sckv_peak_mfma_flops(int kind, int64_t iters, int blocks);

/* Thread-local description of the last failed call ("" if none). */
const char* sckv_peak_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SCKV_PEAK_H_ */
