// Skinny-M fp32 GEMM with B stored transposed (N x K): C = alpha * op(A) B + beta * C
// for M <= 16, the shape of a batch of rows times a weight matrix kept as
// rows of its transpose.
//
// Element (i, j) of the product is row i of op(A) dotted with row j of the
// stored B^T, and both rows are contiguous in k.  So a wave owns JC rows of
// B^T (JC output columns) and streams each of them whole: the 64 lanes read
// 64 consecutive float4 of one row per load (1 KiB runs), U K-chunks of 256
// are in flight, and every lane keeps MR x JC partial dot products.  At the
// end the 64 lanes' partials are added by a butterfly across the wave (the
// shuffle reduction of "GPU compute shaders", How it works: reduce inside a
// group first).  When there are too few columns to fill the GPU, K is also
// split over waves and the slices go through the workspace and the combine
// kernel, added in slice order.
//
// The work is a bandwidth-bound stream over B (AI below 4 FLOP/byte), so it
// runs on the vector ALUs; reshaping it into matrix-core tiles would not
// move the bound.
#include <cstdint>

#include "gemm_f32_internal.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using mfma::load4;

// four floats at a 4-byte aligned address, as one non-temporal 128-bit load
// (multi-dword global loads need dword alignment only)
typedef float floatx4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kWavesPerGroup = 4;
constexpr int kChunk = 256;   // k per wave-wide load: 64 lanes x 4

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

template <int MR, int JC, int U, bool TA>
__global__ void __launch_bounds__(kWavesPerGroup * 64)
    skinny_t_kernel(Problem p, int kslice, int slices, float* __restrict__ part, Epilogue e) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int M = p.M, N = p.N, K = p.K;
  const int j0 = (blockIdx.x * kWavesPerGroup + wave) * JC;
  if (j0 >= N) return;   // the whole wave: no barrier in this kernel
  const int slice = blockIdx.y;
  const int kb = slice * kslice;
  const int ke = min(K, kb + kslice);

  // rows of B^T (clamped: columns past N are computed and dropped)
  const float* brow[JC];
#pragma unroll
  for (int c = 0; c < JC; ++c) brow[c] = p.B + (int64_t)min(j0 + c, N - 1) * p.ldb;
  // element (m, k) of op(A) is arow[m][k * a_ks]; rows past M are clamped
  const int64_t a_ks = TA ? p.lda : 1;
  const float* arow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int mm = min(m, M - 1);
    arow[m] = TA ? p.A + mm : p.A + (int64_t)mm * p.lda;
  }

  float acc[MR][JC];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < JC; ++c) acc[m][c] = 0.f;

  struct Chunk {
    float4 b[JC];
    float4 a[MR];
  };
  // chunk q of this slice: k = kb + 256 q + 4 lane .. + 3, all inside K
  auto load = [&](Chunk& x, int q) {
    const int k = kb + kChunk * q + 4 * lane;
#pragma unroll
    for (int c = 0; c < JC; ++c) {
      const floatx4_a4 v =
          __builtin_nontemporal_load(reinterpret_cast<const floatx4_a4*>(brow[c] + k));
      x.b[c] = make_float4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float* s = arow[m] + (int64_t)k * a_ks;
      x.a[m] = TA ? make_float4(s[0], s[a_ks], s[2 * a_ks], s[3 * a_ks]) : load4(s);
    }
  };
  auto fma_chunk = [&](const Chunk& x) {
#pragma unroll
    for (int c = 0; c < JC; ++c) {
      const float4 b = x.b[c];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        acc[m][c] = fmaf(x.a[m].x, b.x, acc[m][c]);
        acc[m][c] = fmaf(x.a[m].y, b.y, acc[m][c]);
        acc[m][c] = fmaf(x.a[m].z, b.z, acc[m][c]);
        acc[m][c] = fmaf(x.a[m].w, b.w, acc[m][c]);
      }
    }
  };

  // whole chunks, U in flight; a prefetch past the last re-reads the last
  // chunk and is not used (the test is the same for the whole wave)
  const int nq = (ke - kb) / kChunk;
  if (nq > 0) {
    Chunk x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(x[u], min(u, nq - 1));
    for (int q0 = 0; q0 < nq; q0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (q0 + u < nq) fma_chunk(x[u]);
        load(x[u], min(q0 + u + U, nq - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the last partial chunk, element by element
  {
    const int k = kb + kChunk * nq + 4 * lane;
    if (kb + kChunk * nq < ke) {
      float bv[JC][4], av[MR][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = k + e < ke;
        const int kk = ok ? k + e : ke - 1;
#pragma unroll
        for (int c = 0; c < JC; ++c) bv[c][e] = ok ? brow[c][kk] : 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m) av[m][e] = ok ? arow[m][(int64_t)kk * a_ks] : 0.f;
      }
#pragma unroll
      for (int c = 0; c < JC; ++c)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[m][c] = fmaf(av[m][e], bv[c][e], acc[m][c]);
    }
  }

  // add the 64 lanes' partials; lane (m * JC + c) % 64 writes element (m, c)
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int c = 0; c < JC; ++c) {
      const float s = wave_sum(acc[m][c]);
      const int j = j0 + c;
      if (lane == ((m * JC + c) & 63) && m < M && j < N) {
        if (slices == 1) {
          float* d = p.C + (int64_t)m * p.ldc + j;
          *d = epilogue_apply(e, s, d, j);
        } else {
          part[((size_t)slice * M + m) * N + j] = s;
        }
      }
    }
  }
}

// K slices only when the columns alone give too few waves (about 8 per CU
// wanted); each slice a whole number of 256-k chunks, at least 4 of them.
template <int JC>
SkinnyPlan plan_t(const Problem& p, int target) {
  SkinnyPlan pl{};
  const int64_t waves = (p.N + JC - 1) / JC;
  pl.strips = (int)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
  const int64_t chunks = (p.K + kChunk - 1) / kChunk;
  int64_t slices = target > 0 ? target : (2048 + waves - 1) / waves;
  const int64_t cap = chunks / 4 > 1 ? chunks / 4 : 1;
  if (slices > cap) slices = cap;
  if (slices < 1) slices = 1;
  const int64_t per = (chunks + slices - 1) / slices;       // chunks per slice
  pl.splits = (int)((chunks + per - 1) / per);              // no empty slice
  pl.kslice = (int)(per * kChunk);
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.lds_bytes = 0;
  return pl;
}

template <int MR, int JC, int U, bool TA>
hipError_t launch_t(const Problem& p, const SkinnyPlan& pl, float* partials,
                    const Epilogue& e, hipStream_t s) {
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.M > MR || p.batch != 1)
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !partials) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, slices = pl.splits;
  float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &kslice, &slices, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_t_kernel<MR, JC, U, TA>),
      dim3(pl.strips, pl.splits), dim3(kWavesPerGroup * 64), args, 0, s);
  if (err != hipSuccess || pl.splits == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: skinnyt_m<rows>_j<columns per wave>_u<chunks in flight>_<nt|tt>.
#define GEMMF32_SKINNY_T(MR, JC, U)                                                       \
  {"skinnyt_m" #MR "_j" #JC "_u" #U "_nt", MR, kWavesPerGroup, U, true, true, 0, false,  \
   true, &plan_t<JC>, &launch_t<MR, JC, U, false>},                                      \
  {"skinnyt_m" #MR "_j" #JC "_u" #U "_tt", MR, kWavesPerGroup, U, false, true, 0, true,  \
   true, &plan_t<JC>, &launch_t<MR, JC, U, true>}

// The default build holds the kernel the tuning table picks (M <= 8, B^T
// not 16-byte aligned); a build with GEMM_F32_SWEEP also holds the others.
const SkinnyVariant kTVariants[] = {
    {"skinnyt_m8_j4_u2_nt", 8, kWavesPerGroup, 2, true, true, 0, false, true, &plan_t<4>,
     &launch_t<8, 4, 2, false>},
#if GEMM_F32_SWEEP
    {"skinnyt_m8_j4_u2_tt", 8, kWavesPerGroup, 2, false, true, 0, true, true, &plan_t<4>,
     &launch_t<8, 4, 2, true>},
    GEMMF32_SKINNY_T(16, 4, 2),
    GEMMF32_SKINNY_T(8, 8, 2),
    GEMMF32_SKINNY_T(8, 4, 4),
    GEMMF32_SKINNY_T(8, 8, 1),
    GEMMF32_SKINNY_T(8, 4, 3),
    GEMMF32_SKINNY_T(8, 2, 4),
#endif
};

}  // namespace

int skinny_t_variant_count() { return (int)(sizeof(kTVariants) / sizeof(kTVariants[0])); }
const SkinnyVariant& skinny_t_variant(int i) { return kTVariants[i]; }

}  // namespace gemmf32
