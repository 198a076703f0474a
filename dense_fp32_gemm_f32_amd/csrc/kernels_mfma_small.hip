// fp32 GEMM for grids too small to fill the GPU: MFMA fragments loaded
// straight from global memory, and K split over the waves of a workgroup.
//
// A 512^3 product is 1.7 us of MFMA work at peak; with one 64 x 64 tile per
// workgroup it has 64 workgroups, and a K split over workgroups needs a
// second launch for the sum.  Here a workgroup owns a small TM x TN tile (32
// or 64 on a side, so 512^3 gives 256 or 64 workgroups) and its KS waves each
// take a contiguous share of K, computing the whole tile for their share.
// The waves' partial tiles are added in LDS in wave order (a fixed order, so
// reruns give the same bits) and wave 0 writes C with the epilogue.  This is
// the per-group partial + combine of "GPU compute shaders" (How it works)
// inside one workgroup, so a single launch does the product.
//
// Fragments come from global memory (L2 after the first touch: a 512^3
// problem is 2 MiB of A and B), in the lane layout of v_mfma_f32_32x32x2_f32
// with the k-slot permutation of the tiled kernels: for a group of 8 k (four
// MFMA steps), lane l = 32 h + r loads A[m0 + r][8 g + 4 h .. + 3] as one
// 16-byte load and B[8 g + 4 h + s][n0 + r] for s = 0..3 (32 lanes read 128
// consecutive bytes of a row of B); step s multiplies k = 8 g + 4 h + s in
// k-slot h, so each k of the group is used once.  D groups are in flight per
// wave.  Rows past M and columns past N are read at clamped addresses and
// their results are not stored; a partial last group of 8 is read element by
// element with k >= K replaced by zeros.
#include "gemm_f32_internal.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

template <int TM, int TN, int KS>
struct SmallCfg {
  static constexpr int kFM = TM / 32, kFN = TN / 32;
  static constexpr int kAccRegs = kFM * kFN * 16;
  static constexpr int kRedFloats = (KS - 1) * kAccRegs * 64;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32 x 32 MFMA blocks");
  static_assert(kRedFloats * 4 <= 64 * 1024, "the partial tiles must fit the LDS budget");
};

template <int TM, int TN, int KS, int D>
__global__ void __launch_bounds__(KS * 64)
    mfma_small_kernel(Problem p, int tiles_m, int tiles_n, int kchunk, float* part, Epilogue ep) {
  using Cfg = SmallCfg<TM, TN, KS>;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  __shared__ float red[Cfg::kRedFloats > 0 ? Cfg::kRedFloats : 1];

  select_batch(p);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;

  // workgroup -> (K slice across workgroups, tile), as in the tiled kernels
  const int tiles = tiles_m * tiles_n;
  int lin = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int slice = lin / tiles;
  lin -= slice * tiles;
  if (part) {
    const int k0 = slice * kchunk;
    p.A += k0;
    p.B += (int64_t)k0 * p.ldb;
    p.K = min(kchunk, p.K - k0);
    p.C = part + (size_t)slice * p.M * p.N;
    p.ldc = p.N;
  }
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(lin, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * TM, n0 = tn * TN;

  const float* arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = m0 + 32 * i + lr;
    arow[i] = p.A + (int64_t)(r < M ? r : M - 1) * p.lda + 4 * lk;
  }
  const float* bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = n0 + 32 * j + lr;
    bcol[j] = p.B + (int64_t)(4 * lk) * p.ldb + (c < N ? c : N - 1);
  }
  const int64_t ldb = p.ldb;

  // this wave's groups of 8 k: [g_begin, g_end); whole groups end at g_full
  // (a wave past the last group has an empty range and no partial group)
  const int ngroups = (K + 7) / 8;
  const int per = (ngroups + KS - 1) / KS;
  const int g_begin = min(ngroups, wave * per);
  const int g_end = min(ngroups, g_begin + per);
  const int g_full = max(g_begin, min(g_end, K / 8));

  struct Group {
    float4 a[FM];
    float b[4][FN];
  };
  auto load = [&](Group& x, int g) {
    const int k = 8 * g;
#pragma unroll
    for (int i = 0; i < FM; ++i) x.a[i] = load4(arow[i] + k);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) x.b[s][j] = bcol[j][(int64_t)(k + s) * ldb];
  };
  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto compute = [&](const Group& x) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float a = s == 0 ? x.a[i].x : s == 1 ? x.a[i].y : s == 2 ? x.a[i].z : x.a[i].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, x.b[s][j], acc[i][j], 0, 0, 0);
        }
  };

  // whole groups, D in flight: the steady loop refills every buffer, the last
  // two rounds refill only groups that exist
  if (g_full > g_begin) {
    Group buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(buf[d], min(g_begin + d, g_full - 1));
    int g = g_begin;
    for (; g + 2 * D <= g_full; g += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute(buf[d]);
        load(buf[d], g + d + D);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (g + d < g_full) compute(buf[d]);
      if (g + d + D < g_full) load(buf[d], g + d + D);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (g + D + d < g_full) compute(buf[d]);
  }
  // the partial last group (K % 8 != 0), element by element
  if (g_full < g_end) {
    const int k = 8 * g_full + 4 * lk;
    Group x;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float* a = arow[i] + 8 * g_full;
      x.a[i] = make_float4(k < K ? a[0] : 0.f, k + 1 < K ? a[1] : 0.f, k + 2 < K ? a[2] : 0.f,
                           k + 3 < K ? a[3] : 0.f);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        x.b[s][j] = k + s < K ? bcol[j][(int64_t)(8 * g_full + s) * ldb] : 0.f;
    compute(x);
  }

  // ---- the waves' partial tiles, added in wave order -------------------------
  if (KS > 1) {
    if (wave > 0) {
      float* r = red + (wave - 1) * Cfg::kAccRegs * 64;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) r[((i * FN + j) * 16 + q) * 64 + lane] = acc[i][j][q];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < KS; ++w) {
      const float* r = red + (w - 1) * Cfg::kAccRegs * 64;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] += r[((i * FN + j) * 16 + q) * 64 + lane];
    }
  }

  // ---- masked store; a K slice writes its raw partial ------------------------
  store_blocks<FM, FN>(acc, p.C, p.ldc, M, N, m0, n0, lane, part != nullptr, ep);
}

template <int TM, int TN, int KS, int D>
hipError_t launch_small(const Problem& p, int slices, int kchunk, float* partials,
                        const Epilogue& e, hipStream_t s) {
  const int tiles_m = (p.M + TM - 1) / TM;
  const int tiles_n = (p.N + TN - 1) / TN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (slices < 1 || tiles * slices > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch ||
      (slices > 1 && p.batch != 1))
    return hipErrorInvalidConfiguration;
  if (slices > 1) {
    if (!partials || kchunk <= 0 || kchunk % 8 != 0 || (int64_t)(slices - 1) * kchunk >= p.K ||
        (int64_t)slices * kchunk < p.K)
      return hipErrorInvalidValue;
  }
  Problem pp = p;
  int tm = tiles_m, tn = tiles_n, kc = kchunk;
  float* part = slices > 1 ? partials : nullptr;
  Epilogue ee = e;
  void* args[] = {&pp, &tm, &tn, &kc, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_small_kernel<TM, TN, KS, D>),
      dim3((unsigned)(tiles * slices), 1, (unsigned)p.batch), dim3(KS * 64), args, 0, s);
  if (err != hipSuccess || slices == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: mfma_<TM>x<TN>x8_k<waves along K>_g<groups in flight>_small.  The K
// tile (8) is the group of four MFMA steps; the K split across workgroups
// ("_sk_" twins) uses slices of whole groups.
#define GEMMF32_MFMA_SMALL(TM, TN, KS, D)                                               \
  {"mfma_" #TM "x" #TN "x8_k" #KS "_g" #D "_small", TM, TN, 8, TM, TN, true, false, false, \
   &launch_small<TM, TN, KS, D>}

const MfmaVariant kSmallVariants[] = {
    GEMMF32_MFMA_SMALL(32, 32, 4, 4),
#if GEMM_F32_SWEEP
    GEMMF32_MFMA_SMALL(32, 32, 4, 8),
    GEMMF32_MFMA_SMALL(32, 32, 8, 8),
    GEMMF32_MFMA_SMALL(32, 64, 4, 8),
    GEMMF32_MFMA_SMALL(64, 32, 4, 8),
    GEMMF32_MFMA_SMALL(64, 64, 4, 4),
    GEMMF32_MFMA_SMALL(64, 64, 2, 4),
    GEMMF32_MFMA_SMALL(64, 64, 4, 2),
#endif
};

}  // namespace

int mfma_small_variant_count() {
  return (int)(sizeof(kSmallVariants) / sizeof(kSmallVariants[0]));
}
const MfmaVariant& mfma_small_variant(int i) { return kSmallVariants[i]; }

}  // namespace gemmf32
