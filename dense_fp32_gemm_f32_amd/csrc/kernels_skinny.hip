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

// Stream this wave's rows of B and accumulate acc[m][q] += A[m][k] * B[k][col+q].
// FULL: the whole strip is inside N and the whole slice inside K, and B rows
// are 16-byte aligned -- no masks at all.  Otherwise every element is masked.
// The slice of A sits in LDS as rows of `apitch` floats: A[m][kbeg + kl] at
// lds_a[m * apitch + kl]; U is a multiple of 4, so one 128-bit LDS read gives
// four consecutive k of one row (a broadcast: every lane reads the same address).
template <int MR, int U, bool FULL>
__device__ __forceinline__ void skinny_stream(const Problem& p, const float* lds_a, int apitch,
                                              int kbeg, int col, int kl_first, int rows,
                                              float4 (&b0)[U], float (&acc)[MR][4]) {
  const int N = p.N, K = p.K;
  const int64_t ldb = p.ldb;
  const float* bcol = p.B + (col < N ? col : 0);

  auto load_block = [&](float4 (&b)[U], int kl) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gk = kbeg + kl + u;
      const float* src = bcol + (int64_t)gk * ldb;
      if (FULL) {
        b[u] = *reinterpret_cast<const float4*>(src);
      } else {
        const bool kok = gk < K;
        b[u].x = (kok && col + 0 < N) ? src[0] : 0.f;
        b[u].y = (kok && col + 1 < N) ? src[1] : 0.f;
        b[u].z = (kok && col + 2 < N) ? src[2] : 0.f;
        b[u].w = (kok && col + 3 < N) ? src[3] : 0.f;
      }
    }
  };
  auto fma_block = [&](const float4 (&b)[U], int kl) {
#pragma unroll
    for (int u4 = 0; u4 < U; u4 += 4) {
      float4 a[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m)
        a[m] = *reinterpret_cast<const float4*>(&lds_a[m * apitch + kl + u4]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 bv = b[u4 + u];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const float av = u == 0 ? a[m].x : u == 1 ? a[m].y : u == 2 ? a[m].z : a[m].w;
          acc[m][0] = fmaf(av, bv.x, acc[m][0]);
          acc[m][1] = fmaf(av, bv.y, acc[m][1]);
          acc[m][2] = fmaf(av, bv.z, acc[m][2]);
          acc[m][3] = fmaf(av, bv.w, acc[m][3]);
        }
      }
    }
  };

  float4 b1[U];
  for (int r = 0; r < rows; r += 2 * U) {
    load_block(b1, kl_first + r + U);
    fma_block(b0, kl_first + r);
    if (r + 2 * U < rows) load_block(b0, kl_first + r + 2 * U);
    fma_block(b1, kl_first + r + U);
  }
}

// The first block of B rows, issued before A is staged so that its latency
// overlaps the staging.
template <int U, bool FULL>
__device__ __forceinline__ void skinny_first_block(const Problem& p, int kbeg, int col,
                                                   int kl, float4 (&b)[U]) {
  const int N = p.N, K = p.K;
  const float* bcol = p.B + (col < N ? col : 0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int gk = kbeg + kl + u;
    const float* src = bcol + (int64_t)gk * p.ldb;
    if (FULL) {
      b[u] = *reinterpret_cast<const float4*>(src);
    } else {
      const bool kok = gk < K;
      b[u].x = (kok && col + 0 < N) ? src[0] : 0.f;
      b[u].y = (kok && col + 1 < N) ? src[1] : 0.f;
      b[u].z = (kok && col + 2 < N) ? src[2] : 0.f;
      b[u].w = (kok && col + 3 < N) ? src[3] : 0.f;
    }
  }
}

template <int MR, int NW, int U, bool VB>
__global__ void __launch_bounds__(NW * 64)
    skinny_kernel(Problem p, int kslice, int splits, float* __restrict__ part,
                  unsigned* __restrict__ counters) {
  static_assert(U % 4 == 0, "blocks of 4 rows share one 128-bit read of A");
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int s_last;

  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int strip = blockIdx.x, slice = blockIdx.y;
  const int n0 = strip * kStrip;
  const int kbeg = slice * kslice;
  const int rows_w = kslice / NW;          // rows of this slice per wave (multiple of 2U)
  const int kl_first = wave * rows_w;      // first slice-local row of this wave
  const int col = n0 + 4 * lane;
  const bool full = VB && n0 + kStrip <= N && kbeg + kslice <= K;

  float4 b0[U];
  if (full) {
    skinny_first_block<U, true>(p, kbeg, col, kl_first, b0);
  } else {
    skinny_first_block<U, false>(p, kbeg, col, kl_first, b0);
  }

  // ---- this slice of A into LDS, row-major, zero outside M x K ------------
  const int apitch = kslice + 4;
  float* lds_a = lds;
  {
    const int chunks = kslice / 4;
    const bool va = (p.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.A) & 15) == 0);
    for (int e = tid; e < MR * chunks; e += NW * 64) {
      const int m = e / chunks, c = e % chunks;
      const int gk = kbeg + 4 * c;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < M) {
        const float* src = p.A + (int64_t)m * p.lda + gk;
        if (va && gk + 3 < K) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          v.x = gk + 0 < K ? src[0] : 0.f;
          v.y = gk + 1 < K ? src[1] : 0.f;
          v.z = gk + 2 < K ? src[2] : 0.f;
          v.w = gk + 3 < K ? src[3] : 0.f;
        }
      }
      *reinterpret_cast<float4*>(&lds_a[m * apitch + 4 * c]) = v;
    }
  }
  __syncthreads();

  float acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m][0] = acc[m][1] = acc[m][2] = acc[m][3] = 0.f;

  if (full) {
    skinny_stream<MR, U, true>(p, lds_a, apitch, kbeg, col, kl_first, rows_w, b0, acc);
  } else {
    skinny_stream<MR, U, false>(p, lds_a, apitch, kbeg, col, kl_first, rows_w, b0, acc);
  }
  __syncthreads();  // the A slice is no longer read; the LDS is reused below

  // ---- combine the waves: a fixed pairwise tree in LDS ---------------------
  float* red = lds;  // [NW/2][MR][64][4]
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      float* dst = red + (size_t)(wave - half) * MR * 256;
#pragma unroll
      for (int m = 0; m < MR; ++m)
        *reinterpret_cast<float4*>(&dst[m * 256 + 4 * lane]) =
            make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
    }
    __syncthreads();
    if (wave < half) {
      const float* src = red + (size_t)wave * MR * 256;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float4 v = *reinterpret_cast<const float4*>(&src[m * 256 + 4 * lane]);
        acc[m][0] += v.x;
        acc[m][1] += v.y;
        acc[m][2] += v.z;
        acc[m][3] += v.w;
      }
    }
    __syncthreads();
  }
  if (wave == 0) {
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

  // Sum the slices in slice order.  Each thread owns whole (m, n) outputs and
  // loads 8 slices at a time before adding them, so the loads overlap.
  for (int e = tid; e < MR * kStrip; e += NW * 64) {
    const int m = e / kStrip, n = n0 + e % kStrip;
    if (m < M && n < N) {
      const float* src = part + (int64_t)m * N + n;
      const size_t stride = (size_t)M * N;
      float s = 0.f;
      for (int sl0 = 0; sl0 < splits; sl0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = sl0 + j < splits ? src[(size_t)(sl0 + j) * stride] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (sl0 + j < splits) s += v[j];
      }
      p.C[(int64_t)m * p.ldc + n] = s;
    }
  }
  if (tid == 0)
    __hip_atomic_store(&counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- full-K variant: no combine across workgroups -------------------------
//
// A workgroup owns CW columns for the whole of K.  Lane l covers the float4
// column chunk l % (CW/4) and the row group g = l / (CW/4) of the wave; a
// block is 4*G consecutive rows (G row groups, 4 rows each), and the waves of
// the workgroup take blocks in turn.  Each lane reads its four rows of B and
// the matching 4-wide k chunk of every row of A (A is small and stays in L2),
// one block ahead of the arithmetic.  The row groups of a wave are combined
// with a butterfly of lane exchanges, the waves in LDS in wave order, and C is
// written directly: no workspace, no atomics, no fences.
template <int MR, int CW, int NW, int PF, bool VA, bool VB>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MR > 8 ? 2 : 4)))
    skinny_fullk_kernel(Problem p) {
  constexpr int LPR = CW / 4;          // lanes per row (float4 chunks)
  constexpr int G = 64 / LPR;          // row groups per wave
  constexpr int BR = 4 * G;            // rows per block
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "CW in {4..256}, power of two");
  __shared__ __attribute__((aligned(16))) float red[NW][MR][CW];

  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane % LPR, g = lane / LPR;
  const int n0 = blockIdx.x * CW;
  const int col = n0 + 4 * c;
  const bool col4_ok = col + 3 < N;
  const int64_t ldb = p.ldb, lda = p.lda;
  const float* bcol = p.B + (col < N ? col : 0);

  struct Block {
    float4 b[4];
    float4 a[MR];
  };
  // rows kb + 4g .. kb + 4g + 3 of B (this lane's columns) and of every row of A
  auto load = [&](Block& x, int kb) {
    const int k = kb + 4 * g;
    const bool kfull = k + 3 < K;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* src = bcol + (int64_t)(k + u) * ldb;
      if (VB && kfull && col4_ok) {
        x.b[u] = *reinterpret_cast<const float4*>(src);
      } else {
        const bool kok = k + u < K;
        x.b[u].x = (kok && col + 0 < N) ? src[0] : 0.f;
        x.b[u].y = (kok && col + 1 < N) ? src[1] : 0.f;
        x.b[u].z = (kok && col + 2 < N) ? src[2] : 0.f;
        x.b[u].w = (kok && col + 3 < N) ? src[3] : 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      // rows m >= M read row M-1 (valid memory); their sums are never stored
      const float* src = p.A + (int64_t)(m < M ? m : M - 1) * lda + k;
      if (VA && kfull) {
        x.a[m] = *reinterpret_cast<const float4*>(src);
      } else {
        x.a[m].x = k + 0 < K ? src[0] : 0.f;
        x.a[m].y = k + 1 < K ? src[1] : 0.f;
        x.a[m].z = k + 2 < K ? src[2] : 0.f;
        x.a[m].w = k + 3 < K ? src[3] : 0.f;
      }
    }
  };

  float acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m][0] = acc[m][1] = acc[m][2] = acc[m][3] = 0.f;
  auto fma = [&](const Block& x) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float av = u == 0 ? x.a[m].x : u == 1 ? x.a[m].y : u == 2 ? x.a[m].z : x.a[m].w;
        acc[m][0] = fmaf(av, x.b[u].x, acc[m][0]);
        acc[m][1] = fmaf(av, x.b[u].y, acc[m][1]);
        acc[m][2] = fmaf(av, x.b[u].z, acc[m][2]);
        acc[m][3] = fmaf(av, x.b[u].w, acc[m][3]);
      }
    }
  };

  // blocks wave, wave + NW, wave + 2 NW, ...; PF: the next block is loaded
  // while the current one is multiplied, else one block at a time (more waves
  // fit in the register file instead)
  const int nblocks = (K + BR - 1) / BR;
  if (PF) {
    Block x0, x1;
    int blk = wave;
    if (blk < nblocks) load(x0, blk * BR);
    for (; blk < nblocks; blk += 2 * NW) {
      const bool has1 = blk + NW < nblocks;
      if (has1) load(x1, (blk + NW) * BR);
      fma(x0);
      if (blk + 2 * NW < nblocks) load(x0, (blk + 2 * NW) * BR);
      if (has1) fma(x1);
    }
  } else {
    for (int blk = wave; blk < nblocks; blk += NW) {
      Block x;
      load(x, blk * BR);
      fma(x);
    }
  }

  // ---- combine the row groups of the wave (lanes with equal c) -------------
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[m][q] += __shfl_xor(acc[m][q], off, 64);
  }
  // ---- combine the waves in wave order ---------------------------------------
  if (g == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      *reinterpret_cast<float4*>(&red[wave][m][4 * c]) =
          make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
  }
  __syncthreads();
  for (int e = tid; e < MR * CW; e += NW * 64) {
    const int m = e / CW, n = e % CW;
    if (m < M && n0 + n < N) {
      float s = red[0][m][n];
      for (int w = 1; w < NW; ++w) s += red[w][m][n];
      p.C[(int64_t)m * p.ldc + n0 + n] = s;
    }
  }
}

template <int MR, int NW, int U>
SkinnyPlan plan(const Problem& p, int target_splits) {
  SkinnyPlan pl{};
  pl.strips = (p.N + kStrip - 1) / kStrip;
  const int step = NW * 2 * U;   // every wave gets a whole number of block pairs
  int splits = target_splits;
  if (splits <= 0) {
    // about 16 waves per CU in all
    splits = (256 * 16 / NW + pl.strips - 1) / pl.strips;
  }
  // the A slice must fit in 64 KiB of LDS
  const int max_kslice = ((65536 - 1024) / (4 * MR) - 4) / step * step;
  int kslice = (p.K + splits - 1) / splits;
  kslice = (kslice + step - 1) / step * step;
  if (kslice < step) kslice = step;
  if (kslice > max_kslice) kslice = max_kslice;
  pl.kslice = kslice;
  pl.splits = (p.K + kslice - 1) / kslice;
  if (pl.splits < 1) pl.splits = 1;
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.counter_words = pl.splits > 1 ? (size_t)pl.strips : 0;
  const size_t a_bytes = (size_t)MR * (kslice + 4) * 4;          // the A slice
  const size_t red_bytes = (size_t)(NW / 2) * MR * 256 * 4;      // the wave-combine buffer
  pl.lds_bytes = a_bytes > red_bytes ? a_bytes : red_bytes;
  return pl;
}

template <int MR, int NW, int U, bool VB>
hipError_t launch(const Problem& p, const SkinnyPlan& pl, float* partials,
                  unsigned* counters, hipStream_t s) {
  if (pl.splits > 65535 || pl.strips <= 0) return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && (!partials || !counters)) return hipErrorInvalidValue;
  // more than 64 KiB of dynamic LDS must be allowed explicitly, once per kernel
  static const hipError_t attr_err =
      pl.lds_bytes > 65536 - 64
          ? hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<MR, NW, U, VB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024)
          : hipSuccess;
  if (attr_err != hipSuccess) return attr_err;
  Problem pp = p;
  int kslice = pl.kslice, splits = pl.splits;
  void* args[] = {&pp, &kslice, &splits, &partials, &counters};
  return hipLaunchKernel(reinterpret_cast<const void*>(&skinny_kernel<MR, NW, U, VB>),
                         dim3(pl.strips, pl.splits), dim3(NW * 64), args, pl.lds_bytes, s);
}

template <int MR, int CW>
SkinnyPlan plan_fullk(const Problem& p, int) {
  SkinnyPlan pl{};
  pl.splits = 1;
  pl.kslice = p.K;
  pl.strips = (p.N + CW - 1) / CW;
  pl.partial_floats = 0;
  pl.counter_words = 0;
  pl.lds_bytes = 0;
  return pl;
}

template <int MR, int CW, int NW, int PF, bool VA, bool VB>
hipError_t launch_fullk(const Problem& p, const SkinnyPlan& pl, float*, unsigned*,
                        hipStream_t s) {
  if (pl.strips <= 0) return hipErrorInvalidConfiguration;
  Problem pp = p;
  void* args[] = {&pp};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_fullk_kernel<MR, CW, NW, PF, VA, VB>),
                         dim3(pl.strips), dim3(NW * 64), args, 0, s);
}

#define GEMMF32_SKINNY(MR, NW, U, SPL)                                                    \
  {"skinny_m" #MR "_w" #NW "_u" #U "_s" #SPL "_vecb", MR, NW, U, false, true, SPL,        \
   &plan<MR, NW, U>, &launch<MR, NW, U, true>},                                         \
  {"skinny_m" #MR "_w" #NW "_u" #U "_s" #SPL "_scalar", MR, NW, U, false, false, SPL,     \
   &plan<MR, NW, U>, &launch<MR, NW, U, false>}

#define GEMMF32_SKINNY_FULLK(MR, CW, NW, PF)                                              \
  {"skinnyfk_m" #MR "_c" #CW "_w" #NW "_p" #PF "_vec", MR, NW, 0, true, true, 1,          \
   &plan_fullk<MR, CW>, &launch_fullk<MR, CW, NW, PF, true, true>},                       \
  {"skinnyfk_m" #MR "_c" #CW "_w" #NW "_p" #PF "_veca", MR, NW, 0, true, false, 1,        \
   &plan_fullk<MR, CW>, &launch_fullk<MR, CW, NW, PF, true, false>},                      \
  {"skinnyfk_m" #MR "_c" #CW "_w" #NW "_p" #PF "_vecb", MR, NW, 0, false, true, 1,        \
   &plan_fullk<MR, CW>, &launch_fullk<MR, CW, NW, PF, false, true>},                      \
  {"skinnyfk_m" #MR "_c" #CW "_w" #NW "_p" #PF "_scalar", MR, NW, 0, false, false, 1,     \
   &plan_fullk<MR, CW>, &launch_fullk<MR, CW, NW, PF, false, false>}

const SkinnyVariant kVariants[] = {
    GEMMF32_SKINNY(4, 8, 4, 0),
    GEMMF32_SKINNY(8, 8, 4, 0),
    GEMMF32_SKINNY(16, 8, 4, 0),
    GEMMF32_SKINNY(8, 8, 4, 8),
    GEMMF32_SKINNY(8, 4, 4, 16),
    GEMMF32_SKINNY_FULLK(8, 32, 8, 0),
    GEMMF32_SKINNY_FULLK(8, 32, 16, 0),
    GEMMF32_SKINNY_FULLK(8, 16, 8, 0),
    GEMMF32_SKINNY_FULLK(8, 16, 16, 0),
    GEMMF32_SKINNY_FULLK(8, 64, 16, 0),
    GEMMF32_SKINNY_FULLK(4, 32, 16, 0),
    GEMMF32_SKINNY_FULLK(16, 32, 8, 0),
};

}  // namespace

int skinny_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }
const SkinnyVariant& skinny_variant(int i) { return kVariants[i]; }

}  // namespace gemmf32
