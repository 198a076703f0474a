// Macro-tiled fp32 GEMM on the CDNA4 matrix cores (gfx950).
//
// C (M x N) = A (M x K) x B (K x N), row-major, fp32 products and fp32
// accumulation, on v_mfma_f32_32x32x2_f32 (full fp32, no reduced-precision
// input format).
//
// What is kept from the pages' tiled kernels, re-expressed for gfx950:
//  - one workgroup per output tile with a ceil-divided grid ("Optimizing a
//    WebGPU Matmul Kernel using Subgroups", section 2 Workgroups);
//  - adjacent lanes read adjacent addresses (section 3 Global Memory
//    Coalescing) and loads are 128-bit where the rows allow it (section 7
//    Vectorization);
//  - tiles staged through workgroup shared memory (section 4), here LDS,
//    with zero-filled out-of-range elements and a guarded store, as the
//    tiled kernels of the ybb.press page and of the GEMM Optimization Guide
//    (section 4) do;
//  - register blocking of many outputs per thread (sections 5-6) and a
//    hardware matrix instruction for the inner product (section 8 Subgroup
//    Matrix Multiply), here wave64 MFMA accumulators;
//  - shared-memory bank-conflict avoidance (GEMM Optimization Guide,
//    section 6), here XOR swizzles sized for the LDS of gfx950.
// What differs: one barrier per K-tile with a double-buffered LDS (the pages
// use two barriers per tile), a workgroup-to-tile order that keeps
// neighbouring tiles on one XCD's L2, and fp32 MFMA fragments instead of
// 8 x 8 subgroup matrices.
//
// v_mfma_f32_32x32x2_f32 operand layout (wave64, one block):
//   A operand, lane l: A[i = l % 32][k = l / 32]
//   B operand, lane l: B[k = l / 32][j = l % 32]
//   accumulator register r of lane l: D[i = 8*(r/4) + 4*(l/32) + r%4][j = l % 32]
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kGroupM = 8;   // tile rows per raster group

// Workgroups are dealt to the XCDs round-robin by id.  Renumber so that each
// XCD owns one contiguous range of tile ids; neighbouring tiles then share
// that XCD's L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_contiguous_id(int bid, int n) {
  const int q = n / kNumXcd, r = n % kNumXcd;
  const int x = bid % kNumXcd, idx = bid / kNumXcd;
  return x * q + min(x, r) + idx;
}

// Grouped raster: kGroupM tile rows are swept together along N.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = t - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB>
struct Cfg {
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kThreads = kWavesM * kWavesN * 64;
  static constexpr int kFragM = WM / 32;
  static constexpr int kFragN = WN / 32;
  static constexpr int kChunksA = BK / 4;   // float4 chunks per A-tile row
  static constexpr int kChunksB = BN / 4;   // float4 chunks per B-tile row
  static constexpr int kVecA = BM * BK / 4 / kThreads;
  static constexpr int kVecB = BK * BN / 4 / kThreads;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave tiles must divide the tile");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "swizzles need 64-wide tile rows");
  static_assert(BK % 4 == 0 && BK >= 8 && (BK & (BK - 1)) == 0, "BK power of two >= 8");
  static_assert(64 % kChunksA == 0, "a wave covers whole A rows");
  static_assert((BM * BK / 4) % kThreads == 0 && (BK * BN / 4) % kThreads == 0,
                "tile loads divide evenly over the threads");
  // LDS: A stored k-major (A^T tile, m contiguous), B stored k-major (n contiguous).
  static constexpr int kLdsA = BK * BM;
  static constexpr int kLdsB = BK * BN;
};

// XOR swizzle of the m index of the k-major A tile.  The 4-wide k chunk c of
// a global load row lands in its own group of 64/kChunks banks, and rows k
// and k+1 (read together by one MFMA A fragment: lanes 0-31 and 32-63) land
// in opposite halves of the 64 banks.
template <int kChunks>
__device__ __forceinline__ int swz_a(int k) {
  const int c = (k >> 2) & (kChunks - 1);
  return (c ^ ((k & 1) * (kChunks / 2))) * (64 / kChunks);
}
// Rows k and k+1 of the B tile in opposite halves of the 64 banks.
__device__ __forceinline__ int swz_b(int k) { return (k & 1) << 5; }

template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_gemm_kernel(Problem p, int tiles_m, int tiles_n) {
  using C_ = Cfg<BM, BN, BK, WM, WN, VA, VB>;
  __shared__ __attribute__((aligned(16))) float lds_a[2][C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b[2][C_::kLdsB];

  const int tid = threadIdx.x;
  const int M = p.M, N = p.N, K = p.K;

  int tm, tn;
  tile_coords(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global -> register staging ----------------------------------------
  // A: thread loads float4 chunks along k; row = v / kChunksA.
  // B: thread loads float4 chunks along n; row = v / kChunksB.
  const float* a_ptr[C_::kVecA];
  bool a_row_ok[C_::kVecA];
#pragma unroll
  for (int v = 0; v < C_::kVecA; ++v) {
    const int e = tid + v * C_::kThreads;
    const int row = e / C_::kChunksA, kc = (e % C_::kChunksA) * 4;
    const int gr = m0 + row;
    a_row_ok[v] = gr < M;
    a_ptr[v] = p.A + (int64_t)(a_row_ok[v] ? gr : 0) * p.lda + kc;
  }
  const float* b_ptr[C_::kVecB];
  bool b_col_ok[C_::kVecB];  // whole float4 inside N
  int b_ncol[C_::kVecB];     // global column of the chunk
#pragma unroll
  for (int v = 0; v < C_::kVecB; ++v) {
    const int e = tid + v * C_::kThreads;
    const int krow = e / C_::kChunksB, nc = (e % C_::kChunksB) * 4;
    b_ncol[v] = n0 + nc;
    b_col_ok[v] = n0 + nc + 3 < N;
    b_ptr[v] = p.B + (int64_t)krow * p.ldb + (b_ncol[v] < N ? b_ncol[v] : 0);
  }

  float4 ra[C_::kVecA], rb[C_::kVecB];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int v = 0; v < C_::kVecA; ++v) {
      const int e = tid + v * C_::kThreads;
      const int gk = k0 + (e % C_::kChunksA) * 4;
      const float* src = a_ptr[v] + k0;
      if (VA && a_row_ok[v] && gk + 3 < K) {
        ra[v] = *reinterpret_cast<const float4*>(src);
      } else {
        const bool ok = a_row_ok[v];
        ra[v].x = (ok && gk + 0 < K) ? src[0] : 0.f;
        ra[v].y = (ok && gk + 1 < K) ? src[1] : 0.f;
        ra[v].z = (ok && gk + 2 < K) ? src[2] : 0.f;
        ra[v].w = (ok && gk + 3 < K) ? src[3] : 0.f;
      }
    }
#pragma unroll
    for (int v = 0; v < C_::kVecB; ++v) {
      const int e = tid + v * C_::kThreads;
      const int gk = k0 + e / C_::kChunksB;
      const float* src = b_ptr[v] + (int64_t)k0 * p.ldb;
      const bool kok = gk < K;
      if (VB && kok && b_col_ok[v]) {
        rb[v] = *reinterpret_cast<const float4*>(src);
      } else {
        const int nn = b_ncol[v];
        rb[v].x = (kok && nn + 0 < N) ? src[0] : 0.f;
        rb[v].y = (kok && nn + 1 < N) ? src[1] : 0.f;
        rb[v].z = (kok && nn + 2 < N) ? src[2] : 0.f;
        rb[v].w = (kok && nn + 3 < N) ? src[3] : 0.f;
      }
    }
  };

  auto store_tiles = [&](int buf) {
    float* la = lds_a[buf];
    float* lb = lds_b[buf];
#pragma unroll
    for (int v = 0; v < C_::kVecA; ++v) {
      const int e = tid + v * C_::kThreads;
      const int row = e / C_::kChunksA, kc = (e % C_::kChunksA) * 4;
      la[(kc + 0) * BM + (row ^ swz_a<C_::kChunksA>(kc + 0))] = ra[v].x;
      la[(kc + 1) * BM + (row ^ swz_a<C_::kChunksA>(kc + 1))] = ra[v].y;
      la[(kc + 2) * BM + (row ^ swz_a<C_::kChunksA>(kc + 2))] = ra[v].z;
      la[(kc + 3) * BM + (row ^ swz_a<C_::kChunksA>(kc + 3))] = ra[v].w;
    }
#pragma unroll
    for (int v = 0; v < C_::kVecB; ++v) {
      const int e = tid + v * C_::kThreads;
      const int krow = e / C_::kChunksB, nc = (e % C_::kChunksB) * 4;
      *reinterpret_cast<float4*>(&lb[krow * BN + (nc ^ swz_b(krow))]) = rb[v];
    }
  };

  // ---- MFMA work of one wave --------------------------------------------
  const int wave = tid >> 6, lane = tid & 63;
  const int wmi = wave % C_::kWavesM, wni = wave / C_::kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  const int am = wmi * WM + lr;   // + 32 * fragment
  const int bn = wni * WN + lr;

  floatx16 acc[C_::kFragM][C_::kFragN];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < C_::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int buf) {
    const float* la = lds_a[buf];
    const float* lb = lds_b[buf];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const int k = kk + lk;
      float fa[C_::kFragM], fb[C_::kFragN];
#pragma unroll
      for (int i = 0; i < C_::kFragM; ++i)
        fa[i] = la[k * BM + ((am + 32 * i) ^ swz_a<C_::kChunksA>(k))];
#pragma unroll
      for (int j = 0; j < C_::kFragN; ++j)
        fb[j] = lb[k * BN + ((bn + 32 * j) ^ swz_b(k))];
#pragma unroll
      for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < C_::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- K loop: double-buffered LDS, one barrier per K-tile ---------------
  const int ktiles = (K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int t = 0; t < ktiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < ktiles;
    if (more) load_tiles((t + 1) * BK);
    compute(cur);
    if (more) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // ---- masked epilogue ----------------------------------------------------
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i) {
#pragma unroll
    for (int j = 0; j < C_::kFragN; ++j) {
      const int col = n0 + wni * WN + 32 * j + lr;
      const int rbase = m0 + wmi * WM + 32 * i + 4 * lk;
      if (col < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < M) p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB, int kMinWaves>
hipError_t launch(const Problem& p, hipStream_t s) {
  using C_ = Cfg<BM, BN, BK, WM, WN, VA, VB>;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
  Problem pp = p;
  int tm = tiles_m, tn = tiles_n;
  void* args[] = {&pp, &tm, &tn};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_gemm_kernel<BM, BN, BK, WM, WN, VA, VB, kMinWaves>),
      dim3((unsigned)tiles), dim3(C_::kThreads), args, 0, s);
}

#define GEMMF32_MFMA(BM, BN, BK, WM, WN, MW)                                           \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_vec", BM, BN, BK, WM, WN, true, true, \
   &launch<BM, BN, BK, WM, WN, true, true, MW>},                                       \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_veca", BM, BN, BK, WM, WN, true, false,\
   &launch<BM, BN, BK, WM, WN, true, false, MW>},                                      \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_vecb", BM, BN, BK, WM, WN, false, true,\
   &launch<BM, BN, BK, WM, WN, false, true, MW>},                                      \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_scalar", BM, BN, BK, WM, WN, false,  \
   false, &launch<BM, BN, BK, WM, WN, false, false, MW>}

const MfmaVariant kVariants[] = {
    GEMMF32_MFMA(128, 128, 16, 64, 64, 4),
    GEMMF32_MFMA(128, 128, 32, 64, 64, 2),
    GEMMF32_MFMA(64, 64, 16, 32, 32, 4),
};

}  // namespace

int mfma_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }
const MfmaVariant& mfma_variant(int i) { return kVariants[i]; }

}  // namespace gemmf32
