// The pure streaming read of the sweep build (read_probe.hip), for
// measurement: the achievable HBM read rate on this device.
#pragma once

#include <cstdint>

#include "gemm_f32_internal.h"

namespace gemmf32 {

#if GEMM_F32_SWEEP
// Reads x[0 .. n) once: `groups` workgroups of 8 waves, each a contiguous
// chunk of n / groups floats, and writes 8 floats per workgroup to out (the
// per-wave sums of lane 0; out holds 8 groups floats).  Needs n a multiple of
// 256 groups, x 16-byte aligned, 1 <= groups <= 65535.
hipError_t launch_read_probe(const float* x, int64_t n, int groups, float* out, hipStream_t s);
#endif

}  // namespace gemmf32
