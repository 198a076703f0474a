// Measurement only, compiled into the sweep build (-DGEMM_F32_SWEEP=1): a
// pure streaming read of an fp32 array, the rate that the HBM-bound kernels
// of this library (the skinny-M products, the sum) are read against beside
// the 8 TB/s nominal peak.
//
// The pattern is the fastest of the read-only patterns tried on MI355X:
// workgroup g of G reads the contiguous chunk [g c, (g + 1) c) of the array
// (c = n / G), its 8 waves taking 1 KiB pieces w, w + 8, w + 16, ... (one
// 16-byte non-temporal load per lane), four pieces in flight per wave.  Each
// lane adds what it reads; lane 0 of every wave stores its sum to out, so no
// load can be optimised away and the writes are 32 bytes per workgroup.
#include <cstdint>

#include "gemm_f32_internal.h"
#include "read_probe.h"

namespace gemmf32 {

#if GEMM_F32_SWEEP
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWaves = 8;
constexpr int kInFlight = 4;

__global__ void __launch_bounds__(kProbeWaves * 64)
    read_probe_kernel(const float* __restrict__ x, int64_t chunk, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* base = x + (int64_t)blockIdx.x * chunk + 4 * lane;
  const int64_t pieces = chunk / 256;   // 1 KiB pieces of the chunk
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  floatx4 v[kInFlight];
  // piece p of this wave is wave + 8 p; past the end it re-reads the last
  // piece of the chunk and adds nothing
  auto piece = [&](int64_t p) {
    const int64_t q = wave + (int64_t)kProbeWaves * p;
    return __builtin_nontemporal_load(
        reinterpret_cast<const floatx4*>(base + 256 * (q < pieces ? q : pieces - 1)));
  };
  const int64_t mine = (pieces - wave + kProbeWaves - 1) / kProbeWaves;   // pieces of this wave
#pragma unroll
  for (int u = 0; u < kInFlight; ++u) v[u] = piece(u);
  for (int64_t p0 = 0; p0 < mine; p0 += kInFlight) {
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (p0 + u < mine) acc += v[u];
      v[u] = piece(p0 + kInFlight + u);
    }
  }
  if (lane == 0) out[blockIdx.x * kProbeWaves + wave] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

hipError_t launch_read_probe(const float* x, int64_t n, int groups, float* out, hipStream_t s) {
  if (groups < 1 || groups > 65535 || n <= 0 || n % ((int64_t)256 * groups) != 0 ||
      (reinterpret_cast<uintptr_t>(x) & 15) != 0 || !out)
    return hipErrorInvalidValue;
  const float* xx = x;
  int64_t chunk = n / groups;
  float* o = out;
  void* args[] = {&xx, &chunk, &o};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3(groups),
                         dim3(kProbeWaves * 64), args, 0, s);
}
#endif

}  // namespace gemmf32
