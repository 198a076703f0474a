// Fixed scratch memory for gemm_f32_noalloc: a file-scope array in the
// library's device code, so calls through that entry point never allocate.
//
// The array is split in two fixed regions:
//  - exchange slots of the skinny-M kernel that adds its K slices in-kernel.
//    Every kernel that uses slots finds them all zero and leaves them zero,
//    so the region is cleared once per device, before its first use;
//  - per-slice partial sums of the kernels that add their K slices with a
//    second dispatch (written before they are read; never cleared).
// Each device holds its own copy of the array at its own address.  In host
// code the array's name is only a host-side handle: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is passed
// to kernels.  Calls that overlap on one device share the array and race.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/gemm_f32.h"
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

static_assert(GEMM_F32_NOALLOC_SLOT_BYTES % 256 == 0, "slot region keeps 256-byte alignment");

static __device__ __align__(256) unsigned char
    scratch[GEMM_F32_NOALLOC_SLOT_BYTES + GEMM_F32_NOALLOC_PARTIAL_BYTES];

__global__ void __launch_bounds__(256) zero_words(unsigned long long* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0ull;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
unsigned char* g_base[kMaxDevices];   // device address of `scratch`, per device
bool g_ready[kMaxDevices];            // the slot region has been cleared

}  // namespace

int noalloc_scratch(int dev, hipStream_t s, NoallocScratch* out) {
  if (dev < 0 || dev >= kMaxDevices) return GEMM_F32_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ready[dev]) {
    // set-up on this device (current): look up this device's copy of the
    // array, then clear the slot region and wait for it, which needs a
    // stream that is not being captured
    if (!g_base[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return GEMM_F32_ERR_WORKSPACE;
      }
      g_base[dev] = static_cast<unsigned char*>(p);
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_F32_ERR_WORKSPACE;
    }
    if (cap != hipStreamCaptureStatusNone) return GEMM_F32_ERR_WORKSPACE;
    const size_t words = GEMM_F32_NOALLOC_SLOT_BYTES / 8;
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, s,
                       reinterpret_cast<unsigned long long*>(g_base[dev]), words);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_F32_ERR_LAUNCH;
    }
    g_ready[dev] = true;
  }
  out->slots = reinterpret_cast<unsigned long long*>(g_base[dev]);
  out->slot_words = GEMM_F32_NOALLOC_SLOT_BYTES / 8;
  out->partials = reinterpret_cast<float*>(g_base[dev] + GEMM_F32_NOALLOC_SLOT_BYTES);
  out->partial_floats = GEMM_F32_NOALLOC_PARTIAL_BYTES / 4;
  return GEMM_F32_OK;
}

}  // namespace gemmf32
