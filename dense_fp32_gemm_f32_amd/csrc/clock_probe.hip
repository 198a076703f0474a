// The shader clock the GPU sustains under fp32 MFMA load, for measurement
// records: a kernel that keeps every SIMD issuing v_mfma_f32_32x32x2_f32 and
// stamps, per workgroup, the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) after a barrier at its start and
// at its end.  Their ratio over the run is the achieved shader clock; the
// fp32 MFMA peak scales with it (256 FLOP per clock per CU).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// iters x 4 independent 32x32x2 MFMAs per wave (4 accumulator chains keep
// the pipe full); wave 0, lane 0 writes [t0, r0, t1, r1] for its workgroup.
__global__ void __launch_bounds__(256) clock_probe_kernel(int iters,
                                                          unsigned long long* stamps) {
  const float a = 1.0f + 1e-3f * (float)(threadIdx.x & 63);
  const float b = 1.0f - 1e-3f * (float)(threadIdx.x >> 6);
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
  }
  // the chains stay live: their sum is compared with a value it never takes
  const float keep = c0[0] + c1[1] + c2[2] + c3[3];
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    unsigned long long* s = stamps + 4 * (size_t)blockIdx.x;
    s[0] = t0;
    s[1] = r0;
    s[2] = t1;
    s[3] = keep == -1.0f ? 0ull : r1;
  }
}

}  // namespace

hipError_t launch_clock_probe(int iters, unsigned long long* stamps, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(kClockProbeWorkgroups), dim3(256), 0, s, iters,
                     stamps);
  return hipGetLastError();
}

}  // namespace gemmf32
