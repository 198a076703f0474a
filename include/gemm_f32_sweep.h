/*
 * gemm_f32_sweep.h -- the one call that only the sweep build of the library
 * (libgemm_f32_sweep.so, built with -DGEMM_F32_SWEEP=1) exports, beside every
 * call of gemm_f32.h.  It is for measurement: it shows where the time of a
 * launch of one of the macro-tiled kernels goes, workgroup by workgroup.  The
 * pages time whole dispatches ("GPU compute shaders", Performance); this
 * splits one dispatch into its parts.
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

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_SWEEP_H */
