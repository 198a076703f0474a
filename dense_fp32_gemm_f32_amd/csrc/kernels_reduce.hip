// Deterministic sum of an fp32 array: a bandwidth-bound stream, two passes.
//
// "GPU compute shaders" (How it works) reduces an array with one partial sum
// per workgroup -- a grid-stride loop per invocation, then a tree in shared
// memory -- and combines the partials afterwards; its Pitfalls section notes
// that a float sum is bit-identical across runs only if the group count and
// the order are fixed.  Here:
//
//  pass 1: G groups (G and the chunk length depend on n only), group g owns
//          the contiguous chunk [g c, min(n, (g + 1) c)) (c a multiple of 4).
//          Thread t keeps four running sums, one per float4 component, over
//          the float4s t, t + 256, ... of the chunk (16 loads in flight,
//          non-temporal); then (s0 + s1) + (s2 + s3), a butterfly across the
//          wave (xor 32, 16, ..., 1: fp addition commutes, so every lane ends
//          with the same value), and the four waves in LDS in wave order.
//  pass 2: one group adds the G partials the same way and writes *out.
//
// The order of every addition is a function of n alone: with 16-byte aligned
// x the loads are float4, otherwise four scalar loads of the same elements
// feed the same sums, so the result is the same at any address.  Accumulation
// is fp32, as in the pages' kernels.  Any element reaches the result through
// at most d = (ceil(c / 1024) + 11) + (ceil(G / 256) + 8) additions (pass 1:
// its thread's running sum, the tail element, the two component additions,
// six butterfly steps, two wave additions; pass 2 likewise), so the error is
// at most about d 2^-24 sum |x|: 276 2^-24 = 1.7e-5 of sum |x| for n = 2^26.
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;             // 4 waves
constexpr int kUnroll = 16;               // float4 loads in flight per thread (16 KiB per wave)
constexpr int kMaxGroups = 256;           // one per CU of MI355X
constexpr int64_t kMinPerGroup = 16384;   // elements; smaller arrays use fewer groups

__device__ __forceinline__ float block_sum(float s, float* lds) {
  // butterfly across the wave: after the step with distance d, lanes l and
  // l ^ d hold the same value (a + b == b + a), so all 64 lanes end equal
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = s;
  __syncthreads();
  return (lds[0] + lds[1]) + (lds[2] + lds[3]);
}

// four consecutive floats of x at element e (float4 load when VEC)
template <bool VEC>
__device__ __forceinline__ floatx4 load4(const float* x, int64_t e) {
  if (VEC) return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(x + e));
  return floatx4{x[e], x[e + 1], x[e + 2], x[e + 3]};
}

template <bool VEC>
__global__ void __launch_bounds__(kThreads)
    reduce_partial_kernel(const float* __restrict__ x, int64_t n, int64_t chunk,
                          float* __restrict__ part) {
  __shared__ float lds[kThreads / 64];
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t end = begin + chunk < n ? begin + chunk : n;
  const int64_t n4 = (end - begin) >> 2;   // whole float4s of the chunk
  const float* xc = x + begin;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n4; i += kUnroll * kThreads) {
    floatx4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load4<VEC>(xc, 4 * (i + u * kThreads));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += v[u][c];
  }
  for (; i < n4; i += kThreads) {
    const floatx4 v = load4<VEC>(xc, 4 * i);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += v[c];
  }
  // the last (end - begin) % 4 elements (only the last group has any)
  const int64_t rem = (end - begin) - 4 * n4;
  if (threadIdx.x < rem) acc[0] += xc[4 * n4 + threadIdx.x];
  const float s = block_sum((acc[0] + acc[1]) + (acc[2] + acc[3]), lds);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kThreads)
    reduce_final_kernel(const float* __restrict__ part, int groups, float* __restrict__ out) {
  __shared__ float lds[kThreads / 64];
  float s = 0.f;
  for (int i = threadIdx.x; i < groups; i += kThreads) s += part[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) *out = s;
}

}  // namespace

ReducePlan plan_reduce(int64_t n) {
  ReducePlan pl{};
  if (n <= 0) return pl;
  int64_t g = (n + kMinPerGroup - 1) / kMinPerGroup;
  if (g > kMaxGroups) g = kMaxGroups;
  int64_t chunk = (n + g - 1) / g;
  chunk = (chunk + 3) / 4 * 4;
  pl.groups = (int)((n + chunk - 1) / chunk);   // no empty group
  pl.chunk = chunk;
  return pl;
}

hipError_t launch_reduce_sum(int64_t n, const float* x, float* out, float* part,
                             hipStream_t s) {
  const ReducePlan pl = plan_reduce(n);
  if (pl.groups > 0) {
    if (!part) return hipErrorInvalidValue;
    const float* xx = x;
    int64_t nn = n, ch = pl.chunk;
    float* pp = part;
    void* args[] = {&xx, &nn, &ch, &pp};
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    const hipError_t err = hipLaunchKernel(
        vec ? reinterpret_cast<const void*>(&reduce_partial_kernel<true>)
            : reinterpret_cast<const void*>(&reduce_partial_kernel<false>),
        dim3(pl.groups), dim3(kThreads), args, 0, s);
    if (err != hipSuccess) return err;
  }
  const float* pp = part;
  int groups = pl.groups;
  float* o = out;
  void* args[] = {&pp, &groups, &o};
  return hipLaunchKernel(reinterpret_cast<const void*>(&reduce_final_kernel), dim3(1),
                         dim3(kThreads), args, 0, s);
}

}  // namespace gemmf32
