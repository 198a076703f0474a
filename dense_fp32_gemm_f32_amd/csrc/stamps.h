// Instrumented runs of the direct-to-LDS MFMA tiles for measurement: where a
// launch's time goes, per workgroup.  Only the sweep build (-DGEMM_F32_SWEEP=1)
// holds them; the product library has none of this code.
#pragma once

#include <cstdint>

#include "gemm_f32_internal.h"

namespace gemmf32 {

#if GEMM_F32_SWEEP
// Direct-to-LDS tile i (the index into mfma_dma_variant) over the whole K of
// one product, with the update e, as its plain kernel computes it.  Thread 0
// of workgroup w writes stamps[6 w .. 6 w + 5]: the constant 100 MHz counter
// (s_memrealtime) at the workgroup's start, after its K loop (all waves, by a
// barrier) and after its C stores have completed (likewise), then the shader
// cycle counter (s_memtime) at the same three points.  The two barriers and
// the wait are the only additions to the plain kernel's work.  words: the
// length of stamps (at least 6 per tile).  Preconditions as the tile's plain
// launch, no K split.
hipError_t launch_dma_stamped(int i, const Problem& p, const Epilogue& e,
                              unsigned long long* stamps, int64_t words, hipStream_t s);
#endif

}  // namespace gemmf32
