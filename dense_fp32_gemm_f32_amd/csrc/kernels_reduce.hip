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
//          the float4s t, t + 256, ... of the chunk (8 loads in flight,
//          non-temporal); then (s0 + s1) + (s2 + s3), a butterfly across the
//          wave (xor 32, 16, ..., 1: fp addition commutes, so every lane ends
//          with the same value), and the four waves in LDS in wave order.
//  pass 2: the G partials are added the same way, thread t holding partial
//          t, and the sum is written to *out.  Group 0 does this at the end of
//          pass 1, in the same dispatch: every other group posts its partial
//          as one 64-bit word (a flag in the high half, the value in the low
//          half) in exchange slot g with a device-scope atomic store, and
//          thread t of group 0 swaps slot t for zero until it finds the flag,
//          so the value arrives with the flag and no fence is needed, and
//          every slot is left empty.  Only group 0 waits, and on groups that
//          never wait, so the dispatch always completes.  A second dispatch
//          for the G partials measured 4.5 us on its own.
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
constexpr int kInFlight = 8;              // float4 loads in flight per thread (8 KiB per wave)
constexpr int kMaxGroups = 256;           // one per CU of MI355X
constexpr int64_t kMinPerGroup = 16384;   // elements; smaller arrays use fewer groups
constexpr int kMaxPolls = 1 << 20;        // group 0's bound on polling one slot

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

// Pass 1 and, in group 0, pass 2 (groups <= kThreads): group g > 0 posts its
// partial in slots[g]; group 0 collects slots 1 .. groups - 1.
template <bool VEC>
__global__ void __launch_bounds__(kThreads)
    reduce_kernel(const float* __restrict__ x, int64_t n, int64_t chunk,
                  unsigned long long* __restrict__ slots, float* __restrict__ out) {
  __shared__ float lds[kThreads / 64];
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t end = begin + chunk < n ? begin + chunk : n;
  const int64_t n4 = (end - begin) >> 2;   // whole float4s of the chunk
  const float* xc = x + begin;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // float4 j of thread t is t + 256 j of the chunk, added in order j = 0,
  // 1, ...; the load of float4 j + kInFlight is issued right after float4 j
  // is added, so the loads stay in flight without bursts (past the end of
  // the chunk they re-read its last float4, which is not added)
  const int64_t tid = threadIdx.x;
  const int64_t cnt = n4 > tid ? (n4 - tid + kThreads - 1) / kThreads : 0;
  if (cnt > 0) {
    auto load_j = [&](int64_t j) {
      const int64_t e = tid + j * kThreads;
      return load4<VEC>(xc, 4 * (e < n4 ? e : n4 - 1));
    };
    floatx4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = load_j(u);
    for (int64_t j0 = 0; j0 < cnt; j0 += kInFlight) {
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        if (j0 + u < cnt) {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += v[u][c];
        }
        v[u] = load_j(j0 + kInFlight + u);
      }
    }
  }
  // the last (end - begin) % 4 elements (only the last group has any)
  const int64_t rem = (end - begin) - 4 * n4;
  if (threadIdx.x < rem) acc[0] += xc[4 * n4 + threadIdx.x];
  const float part = block_sum((acc[0] + acc[1]) + (acc[2] + acc[3]), lds);
  if (blockIdx.x != 0) {
    if (threadIdx.x == 0)
      __hip_atomic_store(slots + blockIdx.x, (1ull << 32) | __float_as_uint(part),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // group 0: thread t takes partial t (its own for t = 0), then the same sum
  // as for any pass-1 thread values
  float s = 0.f;
  const int t = threadIdx.x;
  if (t == 0) {
    s += part;
  } else if (t < (int)gridDim.x) {
    // The other groups never wait, so their partials arrive within the time
    // of the stream; the bound on polling (about 1-2 s at one atomic round
    // trip per poll) only guarantees that the dispatch ends, with NaN as the
    // sum, should a partial not arrive.  A partial that arrives after that
    // stays in its slot until the workspaces are released.
    unsigned long long w = 0;
    for (int poll = 0; poll < kMaxPolls; ++poll) {
      w = __hip_atomic_exchange(slots + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((w >> 32) != 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
    s += (w >> 32) != 0 ? __uint_as_float((unsigned)w) : __builtin_nanf("");
  }
  __syncthreads();   // every wave has read lds in the block_sum above
  s = block_sum(s, lds);
  if (t == 0) *out = s;
}

// n == 0: the empty sum, +0.
__global__ void reduce_empty_kernel(float* __restrict__ out) {
  if (threadIdx.x == 0) *out = 0.f;
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

hipError_t launch_reduce_sum(int64_t n, const float* x, float* out, unsigned long long* slots,
                             hipStream_t s) {
  const ReducePlan pl = plan_reduce(n);
  if (pl.groups == 0) {
    float* o = out;
    void* args[] = {&o};
    return hipLaunchKernel(reinterpret_cast<const void*>(&reduce_empty_kernel), dim3(1), dim3(64),
                           args, 0, s);
  }
  if (pl.groups > kThreads || (pl.groups > 1 && !slots)) return hipErrorInvalidValue;
  const float* xx = x;
  int64_t nn = n, ch = pl.chunk;
  unsigned long long* sl = slots;
  float* o = out;
  void* args[] = {&xx, &nn, &ch, &sl, &o};
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  return hipLaunchKernel(vec ? reinterpret_cast<const void*>(&reduce_kernel<true>)
                             : reinterpret_cast<const void*>(&reduce_kernel<false>),
                         dim3(pl.groups), dim3(kThreads), args, 0, s);
}

}  // namespace gemmf32
