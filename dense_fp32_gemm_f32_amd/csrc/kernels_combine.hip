// Sum of K-slice partial products into C.
//
// When K is split over workgroups, each slice writes its partial product
// into its own M x N buffer and a second dispatch adds them.  This is the
// "combine groups" step of "GPU compute shaders" (How it works, step 6: one
// partial per group, reduced in a second pass).  The slices are added in a
// fixed order, so a rerun gives bitwise the same C, as the Pitfalls section
// of that page asks.
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;
constexpr int kColsPerBlock = kThreads * kPerThread;
constexpr int kMaxGridY = 65535;

// C[m][n] = alpha * (part[0][m][n] + part[1][m][n] + ...) + beta * C[m][n],
// the slices added in slice order (C not read when beta == 0), with part
// packed (pitch N) and slice s at part + s*M*N.  Block (x, y) covers columns
// [1024 x, 1024 x + 1024) of rows y, y + gridDim.y, ...; a thread owns four
// consecutive columns, loaded as one 16-byte chunk per slice when N is a
// multiple of 4 (then every row of every slice starts 16-byte aligned).
__global__ void __launch_bounds__(kThreads) combine_kernel(Problem p, int slices,
                                                          const float* __restrict__ part,
                                                          Epilogue e) {
  const int N = p.N;
  const int n0 = blockIdx.x * kColsPerBlock + kPerThread * threadIdx.x;
  if (n0 >= N) return;
  const bool vec = (N % 4) == 0;
  const size_t slice_stride = (size_t)p.M * N;
  for (int m = blockIdx.y; m < p.M; m += gridDim.y) {
    const float* row = part + (size_t)m * N + n0;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < slices; s0 += 4) {
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* src = row + (size_t)(s0 + j) * slice_stride;
        if (s0 + j >= slices) {
          v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        } else if (vec) {
          v[j] = *reinterpret_cast<const float4*>(src);
        } else {
          v[j].x = src[0];
          v[j].y = n0 + 1 < N ? src[1] : 0.f;
          v[j].z = n0 + 2 < N ? src[2] : 0.f;
          v[j].w = n0 + 3 < N ? src[3] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (s0 + j < slices) {
          s[0] += v[j].x;
          s[1] += v[j].y;
          s[2] += v[j].z;
          s[3] += v[j].w;
        }
      }
    }
    float* dst = p.C + (int64_t)m * p.ldc + n0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      if (n0 + q < N) {
        dst[q] = epilogue_apply(e, s[q], dst + q, (int64_t)n0 + q);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const Problem& p, int slices, const float* partials, hipStream_t s,
                          const Epilogue& e) {
  if (slices < 1 || !partials) return hipErrorInvalidValue;
  if (p.batch != 1) return hipErrorInvalidConfiguration;
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const unsigned bx = (unsigned)((p.N + kColsPerBlock - 1) / kColsPerBlock);
  const unsigned by = (unsigned)(p.M < kMaxGridY ? p.M : kMaxGridY);
  Problem pp = p;
  int sl = slices;
  const float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &sl, &part, &ee};
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3(bx, by),
                         dim3(kThreads), args, 0, s);
}

}  // namespace gemmf32
