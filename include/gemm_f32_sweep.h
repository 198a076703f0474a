/*
 * gemm_f32_sweep.h -- the calls that only the sweep build of the library
 * (libgemm_f32_sweep.so, built with -DGEMM_F32_SWEEP=1) exports, beside every
 * call of gemm_f32.h.  Both are for measurement.  gemm_f32_stamped shows
 * where the time of a launch of one of the macro-tiled kernels goes,
 * workgroup by workgroup: the pages time whole dispatches ("GPU compute
 * shaders", Performance), and this splits one dispatch into its parts.
 * gemm_f32_read_probe gives the HBM read rate that the bandwidth-bound
 * kernels can be held against, beside the nominal peak.
 */
#ifndef GEMM_F32_SWEEP_H
#define GEMM_F32_SWEEP_H

#include <stdint.h>

#include "gemm_f32.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gemm_f32_stamped -- C = A x B as gemm_f32_run_kernel(index, ...) computes
 * it, with an instrumented copy of that kernel.  index must name one of the
 * direct-to-LDS macro-tiled entries (names "mfma_*_d6_vec"); the arguments
 * must be ones that entry accepts, with M, N and K positive.  The copy adds
 * two workgroup barriers and one wait for the C stores, and thread 0 of
 * workgroup w writes six 64-bit words to stamps[6w .. 6w + 5]:
 *   0, 1, 2: the constant-rate counter (s_memrealtime; rate from
 *            hipDeviceAttributeWallClockRate, 100 MHz on MI355X) at the
 *            workgroup's start, after the K loop of all its waves, and after
 *            all its C stores have completed;
 *   3, 4, 5: the shader cycle counter (s_memtime) at the same points.
 * Workgroup w is launch index w (blockIdx.x); its tile is the one the plain
 * kernel gives that index.  stamps: device memory of stamp_words >= 6 x (the
 * tile count) uint64, caller-owned, 8-byte aligned.  Errors: index not such
 * an entry, an empty product or arguments it does not accept
 * GEMM_F32_ERR_BAD_KERNEL; the argument checks of gemm_f32; NULL stamps
 * GEMM_F32_ERR_NULL_PTR; misaligned or unreachable stamps
 * GEMM_F32_ERR_POINTER; too few words GEMM_F32_ERR_INVALID_DIM.  Asynchronous
 * on `stream` like gemm_f32.
 */
int gemm_f32_stamped(int index, int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     unsigned long long *stamps, int64_t stamp_words,
                     void *stream);

/*
 * gemm_f32_read_probe -- reads the n floats of x once, with the fastest pure
 * read pattern found for MI355X: `groups` workgroups of 8 waves, workgroup g
 * streaming the contiguous chunk x[g c .. (g + 1) c) with c = n / groups in
 * 1 KiB pieces (16-byte non-temporal loads, four pieces in flight per wave).
 * It writes 8 floats per workgroup to out (sums of what lane 0 of each wave
 * read, so that no load is dead), nothing else.  x: device memory, 16-byte
 * aligned, n a multiple of 256 * groups; out: 8 * groups floats of device
 * memory, not overlapping x; both caller-owned.  Errors: groups outside
 * [1, 65535], n <= 0, above 2^40 or not such a multiple
 * GEMM_F32_ERR_INVALID_DIM; NULL x or out GEMM_F32_ERR_NULL_PTR; x not
 * 16-byte aligned, out not 4-byte aligned, or either unreachable
 * GEMM_F32_ERR_POINTER; out overlapping x GEMM_F32_ERR_ALIAS; then the device
 * check of gemm_f32.  Asynchronous on `stream`.
 */
int gemm_f32_read_probe(const float *x, int64_t n, int groups, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_SWEEP_H */
