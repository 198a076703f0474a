// The naive reference kernel and the K == 0 fill (C = beta * C).
//
// Reference kernel: one thread per element of C, as in section 1 (Naive) of
// "Optimizing a WebGPU Matmul Kernel using Subgroups", with 16 x 16
// workgroups and a ceil-divided grid (section 2) and the column index on the
// fastest-varying thread dimension so that adjacent lanes read adjacent B
// columns (section 3).  Out-of-range threads return, as in the guarded naive
// kernels of the ybb.press page and of "WebGPU 行列積の限界を測る".  The sum runs
// over k in ascending order with fp32 fused multiply-add.
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

constexpr int kRefTile = 16;
constexpr int kMaxGridY = 65535;

__global__ void __launch_bounds__(kRefTile * kRefTile) ref_gemm_kernel(Problem p) {
  select_batch(p);
  const int col = blockIdx.x * kRefTile + threadIdx.x;
  if (col >= p.N) return;
  // grid-stride over rows when M needs more than kMaxGridY row tiles
  for (int64_t row = (int64_t)blockIdx.y * kRefTile + threadIdx.y; row < p.M;
       row += (int64_t)gridDim.y * kRefTile) {
    const float* a = p.A + row * p.lda;
    const float* b = p.B + col;
    float sum = 0.f;
    for (int k = 0; k < p.K; ++k) sum = fmaf(a[k], b[(int64_t)k * p.ldb], sum);
    p.C[row * p.ldc + col] = sum;
  }
}

// An empty sum (K == 0): C = beta * C, or +0.0 without reading C when beta == 0.
__global__ void __launch_bounds__(256) scale_kernel(Problem p, Epilogue e) {
  select_batch(p);
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= p.N) return;
  for (int64_t row = blockIdx.y; row < p.M; row += gridDim.y) {
    float* c = p.C + row * p.ldc + col;
    *c = epilogue_apply(e, 0.f, c, col);
  }
}

}  // namespace

hipError_t launch_ref(const Problem& p, hipStream_t s) {
  if (p.batch < 1 || p.batch > kMaxLaunchBatch) return hipErrorInvalidConfiguration;
  const int64_t gx = (p.N + kRefTile - 1) / kRefTile;
  int64_t gy = (p.M + kRefTile - 1) / kRefTile;
  if (gy > kMaxGridY) gy = kMaxGridY;
  Problem pp = p;
  void* args[] = {&pp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&ref_gemm_kernel),
                         dim3((unsigned)gx, (unsigned)gy, (unsigned)p.batch),
                         dim3(kRefTile, kRefTile), args, 0, s);
}

hipError_t launch_scale(const Problem& p, const Epilogue& e, hipStream_t s) {
  if (p.batch < 1 || p.batch > kMaxLaunchBatch) return hipErrorInvalidConfiguration;
  const int64_t gx = (p.N + 255) / 256;
  int64_t gy = p.M;
  if (gy > kMaxGridY) gy = kMaxGridY;
  Problem pp = p;
  Epilogue ee = e;
  void* args[] = {&pp, &ee};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scale_kernel),
                         dim3((unsigned)gx, (unsigned)gy, (unsigned)p.batch), dim3(256), args,
                         0, s);
}

}  // namespace gemmf32
