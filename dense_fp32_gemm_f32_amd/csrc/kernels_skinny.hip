// Skinny-M fp32 GEMM (M <= 16): a bandwidth-bound stream over B.
//
// With few rows of A, every element of B is used only M times, so the time
// goes into reading B once from HBM.  Each workgroup owns a strip of 256
// columns (64 lanes x float4, coalesced 1 KiB per B row) and one slice of K;
// its waves split the slice further.  The partial sums are combined in a
// fixed order, never with floating-point atomics, so reruns are bitwise
// identical.  This follows the "combine groups" step of "GPU compute
// shaders" (How it works, step 6: one partial per group, then a reduction)
// and its reproducibility pitfall (a float sum depends on the group count and
// order, so both are fixed here); the tree of its reduction example becomes
// an in-order sum over waves in LDS and over K slices in the workspace.
//
// Combining the K slices: each workgroup writes its partial sums to the
// workspace, then bumps the strip's arrival counter.  The workgroup that
// arrives last sums the slices in slice order 0, 1, ..., S-1, writes C and
// resets the counter to zero for the next call.  One launch, no second pass.
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

constexpr int kStrip = 256;   // columns per workgroup

template <int MR, int NW, int U, bool VB>
__global__ void __launch_bounds__(NW * 64)
    skinny_kernel(Problem p, int kslice, int splits, float* __restrict__ part,
                  unsigned* __restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int s_last;

  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int strip = blockIdx.x, slice = blockIdx.y;
  const int n0 = strip * kStrip;
  const int kbeg = slice * kslice;

  // ---- this slice of A, k-major, rows >= M and k >= K zero ----------------
  float* lds_a = lds;  // [kslice][MR]
  for (int e = tid; e < kslice * MR; e += NW * 64) {
    const int m = e / kslice, kl = e % kslice;
    const int gk = kbeg + kl;
    lds_a[kl * MR + m] = (m < M && gk < K) ? p.A[(int64_t)m * p.lda + gk] : 0.f;
  }
  __syncthreads();

  // ---- stream B: wave w takes row blocks w, w+NW, ... of U rows -----------
  const int col = n0 + 4 * lane;
  const bool col4_ok = col + 3 < N;
  const float* bcol = p.B + (col < N ? col : 0);
  float acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m][0] = acc[m][1] = acc[m][2] = acc[m][3] = 0.f;

  const int nblocks = kslice / U;
  for (int blk = wave; blk < nblocks; blk += NW) {
    const int kl0 = blk * U;
    float4 b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gk = kbeg + kl0 + u;
      const float* src = bcol + (int64_t)gk * p.ldb;
      if (VB && gk < K && col4_ok) {
        b[u] = *reinterpret_cast<const float4*>(src);
      } else {
        const bool kok = gk < K;
        b[u].x = (kok && col + 0 < N) ? src[0] : 0.f;
        b[u].y = (kok && col + 1 < N) ? src[1] : 0.f;
        b[u].z = (kok && col + 2 < N) ? src[2] : 0.f;
        b[u].w = (kok && col + 3 < N) ? src[3] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* arow = lds_a + (kl0 + u) * MR;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float a = arow[m];
        acc[m][0] = fmaf(a, b[u].x, acc[m][0]);
        acc[m][1] = fmaf(a, b[u].y, acc[m][1]);
        acc[m][2] = fmaf(a, b[u].z, acc[m][2]);
        acc[m][3] = fmaf(a, b[u].w, acc[m][3]);
      }
    }
  }

  // ---- combine the waves in order: ((w0 + w1) + w2) + ... ----------------
  __syncthreads();  // the A slice is no longer read; reuse the LDS
  float* red = lds;  // [NW-1][MR][64][4]
  if (wave > 0) {
    float* dst = red + (size_t)(wave - 1) * MR * 256;
#pragma unroll
    for (int m = 0; m < MR; ++m)
      *reinterpret_cast<float4*>(&dst[m * 256 + 4 * lane]) =
          make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < NW; ++w) {
      const float* src = red + (size_t)(w - 1) * MR * 256;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float4 v = *reinterpret_cast<const float4*>(&src[m * 256 + 4 * lane]);
        acc[m][0] += v.x;
        acc[m][1] += v.y;
        acc[m][2] += v.z;
        acc[m][3] += v.w;
      }
    }
    float* out;
    int64_t ld;
    if (splits == 1) {
      out = p.C;
      ld = p.ldc;
    } else {
      out = part + (size_t)slice * M * N;
      ld = N;
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < N) out[(int64_t)m * ld + col + q] = acc[m][q];
      }
    }
  }
  if (splits == 1) return;

  // ---- the last workgroup of the strip sums the slices in order ---------
  __threadfence();  // release this workgroup's partial sums device-wide
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&counters[strip], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire the other workgroups' partial sums

  for (int e = tid; e < MR * kStrip; e += NW * 64) {
    const int m = e / kStrip, n = n0 + e % kStrip;
    if (m < M && n < N) {
      const float* src = part + (int64_t)m * N + n;
      float s = 0.f;
      for (int sl = 0; sl < splits; ++sl) s += src[(size_t)sl * M * N];
      p.C[(int64_t)m * p.ldc + n] = s;
    }
  }
  if (tid == 0)
    __hip_atomic_store(&counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MR, int NW, int U>
SkinnyPlan plan(const Problem& p, int target_splits) {
  SkinnyPlan pl{};
  pl.strips = (p.N + kStrip - 1) / kStrip;
  const int step = NW * U;
  int splits = target_splits;
  if (splits <= 0) {
    // enough workgroups to give every CU two, within the LDS limit below
    splits = (512 + pl.strips - 1) / pl.strips;
  }
  // the A slice must fit the LDS budget: kslice * MR floats <= 48 KiB
  const int max_kslice = (49152 / (4 * MR)) / step * step;
  int kslice = (p.K + splits - 1) / splits;
  kslice = (kslice + step - 1) / step * step;
  if (kslice < step) kslice = step;
  if (kslice > max_kslice) kslice = max_kslice;
  pl.kslice = kslice;
  pl.splits = (p.K + kslice - 1) / kslice;
  if (pl.splits < 1) pl.splits = 1;
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.counter_words = pl.splits > 1 ? (size_t)pl.strips : 0;
  const size_t a_bytes = (size_t)kslice * MR * 4;
  const size_t red_bytes = (size_t)(NW - 1) * MR * 256 * 4;
  pl.lds_bytes = a_bytes > red_bytes ? a_bytes : red_bytes;
  return pl;
}

template <int MR, int NW, int U, bool VB>
hipError_t launch(const Problem& p, const SkinnyPlan& pl, float* partials,
                  unsigned* counters, hipStream_t s) {
  if (pl.splits > 65535 || pl.strips <= 0) return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && (!partials || !counters)) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, splits = pl.splits;
  void* args[] = {&pp, &kslice, &splits, &partials, &counters};
  return hipLaunchKernel(reinterpret_cast<const void*>(&skinny_kernel<MR, NW, U, VB>),
                         dim3(pl.strips, pl.splits), dim3(NW * 64), args, pl.lds_bytes, s);
}

#define GEMMF32_SKINNY(MR, NW, U, SPL)                                                    \
  {"skinny_m" #MR "_w" #NW "_u" #U "_s" #SPL "_vec", MR, NW, U, true, SPL,               \
   &plan<MR, NW, U>, &launch<MR, NW, U, true>},                                         \
  {"skinny_m" #MR "_w" #NW "_u" #U "_s" #SPL "_scalar", MR, NW, U, false, SPL,           \
   &plan<MR, NW, U>, &launch<MR, NW, U, false>}

const SkinnyVariant kVariants[] = {
    GEMMF32_SKINNY(4, 4, 8, 0),
    GEMMF32_SKINNY(8, 4, 8, 0),
    GEMMF32_SKINNY(16, 4, 4, 0),
    GEMMF32_SKINNY(8, 4, 8, 16),
    GEMMF32_SKINNY(8, 8, 4, 8),
};

}  // namespace

int skinny_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }
const SkinnyVariant& skinny_variant(int i) { return kVariants[i]; }

}  // namespace gemmf32
