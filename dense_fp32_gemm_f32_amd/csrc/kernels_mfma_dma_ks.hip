// Macro-tiled fp32 GEMM on the CDNA4 matrix cores with direct global -> LDS
// loads and every K-tile shared between KS waves per wave tile (gfx950).
//
// Tile, LDS layout, swizzles, fragment reads and MFMA order are those of the
// direct-to-LDS kernel in kernels_mfma_dma.hip.  There a 64 x 64 tile runs
// four waves of 32 x 32, one per SIMD, and a wave stalls whenever it issues
// its share of the next tile's loads or waits at the barrier, with no other
// wave on its SIMD to fill the MFMA pipe.  Here KS waves own each wave tile
// and take KS contiguous shares of the 8-k groups of every K-tile (wave group
// g: groups g G, ..., g G + G - 1 with G = BK / 8 / KS), so each SIMD holds
// KS waves whose load issue, LDS reads and barrier waits overlap each other's
// MFMAs; the MFMA work per SIMD is unchanged.  All waves share the loads of
// a tile.  After the K loop, groups 1 .. KS - 1 leave their partial tiles in
// LDS and group 0 adds them in group order (a fixed order: reruns give the
// same bits) and stores C through the masked epilogue.
//
// Preconditions (checked by the dispatcher, as for the other direct-to-LDS
// kernel): A and B 16-byte aligned, lda, ldb and N multiples of 4, K a
// multiple of BK.  Rows of A past M and columns of B past N are read at
// clamped addresses and only reach rows and columns of C that are not
// stored.
#include <cstdint>
#include <type_traits>

#include "gemm_f32_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

template <int BM, int BN, int BK, int WM, int WN, int KS>
struct KsCfg {
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kTileWaves = kWavesM * kWavesN;   // waves of one K share
  static constexpr int kWaves = kTileWaves * KS;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kFragM = WM / 32;
  static constexpr int kFragN = WN / 32;
  static constexpr int kChunksA = BK / 4;   // float4 chunks per A-tile row
  static constexpr int kChunksB = BN / 4;   // float4 chunks per B-tile row
  static constexpr int kVecA = BM * BK / 4 / kThreads;
  static constexpr int kVecB = BK * BN / 4 / kThreads;
  static constexpr int kGroups = BK / 8;           // 8-k groups per K-tile
  static constexpr int kMyGroups = kGroups / KS;   // groups per wave
  static constexpr int kLdsA = BM * BK;
  static constexpr int kLdsB = BK * BN;
  static constexpr int kRed = (KS - 1) * kTileWaves * kFragM * kFragN * 16 * 64;
  static_assert(KS == 2 || KS == 4, "two or four K shares");
  static_assert(BM % WM == 0 && BN % WN == 0, "wave tiles must divide the tile");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(BN % 64 == 0, "the B swizzle needs 64-wide tile rows");
  static_assert(BK == 32 || BK == 64, "BK in {32, 64}");
  static_assert(kGroups % KS == 0 && kMyGroups % 2 == 0,
                "each wave takes an even number of whole 8-k groups");
  static_assert((BM * BK / 4) % kThreads == 0 && (BK * BN / 4) % kThreads == 0,
                "tile loads divide evenly over the threads");
};

// The K loop of one wave: its share (groups q0 .. q0 + kMyGroups - 1) of
// every K-tile, with its share of every tile's loads.
template <int BM, int BN, int BK, int WM, int WN, int KS>
__device__ __forceinline__ void ks_k_loop(
    float* lds_a0, float* lds_b0, float* lds_a1, float* lds_b1,
    const float* const (&a_src)[KsCfg<BM, BN, BK, WM, WN, KS>::kVecA],
    const float* const (&b_src)[KsCfg<BM, BN, BK, WM, WN, KS>::kVecB], int64_t ldb, int wave,
    int lane, int ktiles, floatx16 (&acc)[WM / 32][WN / 32]) {
  using C_ = KsCfg<BM, BN, BK, WM, WN, KS>;
  constexpr int kTileLoads = C_::kVecA + C_::kVecB;
  auto dma_one = [&](float* la, float* lb, int k0, int idx) {
    if (idx < C_::kVecA) {
      load_lds16(a_src[idx] + k0, la + (idx * C_::kWaves + wave) * 256);
    } else {
      const int v = idx - C_::kVecA;
      load_lds16(b_src[v] + (int64_t)k0 * ldb, lb + (v * C_::kWaves + wave) * 256);
    }
  };

  const int kg = wave / C_::kTileWaves, tw = wave % C_::kTileWaves;
  const int q0 = kg * C_::kMyGroups;   // first 8-k group of this wave's share
  const int wmi = tw % C_::kWavesM, wni = tw / C_::kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  int a_off[C_::kFragM][C_::kMyGroups];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i) {
    const int row = wmi * WM + 32 * i + lr;
#pragma unroll
    for (int qi = 0; qi < C_::kMyGroups; ++qi)
      a_off[i][qi] = row * BK + 4 * ((2 * (q0 + qi) + lk) ^ swz_a<C_::kChunksA>(row));
  }
  int b_off[C_::kFragN];
#pragma unroll
  for (int j = 0; j < C_::kFragN; ++j) b_off[j] = (wni * WN + 32 * j + lr) ^ (lk << 5);

  struct Frag {
    float4 a[C_::kFragM];
    float b[4][C_::kFragN];
  };
  auto read_one = [&](Frag& f, const float* la, const float* lb, int qi, int idx) {
    if (idx < C_::kFragM) {
      f.a[idx] = *reinterpret_cast<const float4*>(&la[a_off[idx][qi]]);
    } else {
      const int j = (idx - C_::kFragM) / 2, s0 = 2 * ((idx - C_::kFragM) % 2);
      const int krow = 8 * (q0 + qi) + 4 * lk + s0;
      f.b[s0][j] = lb[krow * BN + b_off[j]];
      f.b[s0 + 1][j] = lb[(krow + 1) * BN + b_off[j]];
    }
  };
  // a wave tile of one 32 x 32 block chains every MFMA on one accumulator;
  // there the odd k-steps go to a second one, added after the loop
  constexpr bool kDual = C_::kFragM * C_::kFragN == 1;
  floatx16 acc_odd = {};
  auto mfma_one = [&](const Frag& f, int idx) {
    const int s = idx / (C_::kFragM * C_::kFragN);
    const int i = (idx / C_::kFragN) % C_::kFragM, j = idx % C_::kFragN;
    const float a = s == 0 ? f.a[i].x : s == 1 ? f.a[i].y : s == 2 ? f.a[i].z : f.a[i].w;
    if constexpr (kDual) {
      if (s & 1) {
        acc_odd = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.b[s][j], acc_odd, 0, 0, 0);
        return;
      }
    }
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.b[s][j], acc[i][j], 0, 0, 0);
  };

  constexpr int kMfmaPerGroup = 4 * C_::kFragM * C_::kFragN;
  constexpr int kHalf = kMfmaPerGroup / 2;
  constexpr int kReadsPerGroup = C_::kFragM + 2 * C_::kFragN;
  constexpr int kReadsPer = (kReadsPerGroup + kHalf - 1) / kHalf;
  constexpr int kLoadsPer = (kTileLoads + kHalf - 1) / kHalf;

  // Every step has the same branch-free shape: the loads of a tile past the
  // end re-read the last tile into the buffer that is no longer needed, and
  // the last step reads fragments it will not use.
  const int last_k0 = (ktiles - 1) * BK;
  Frag f0, f1;
#pragma unroll
  for (int idx = 0; idx < kTileLoads; ++idx) dma_one(lds_a0, lds_b0, 0, idx);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int idx = 0; idx < kReadsPerGroup; ++idx) read_one(f0, lds_a0, lds_b0, 0, idx);
#pragma unroll
  for (int idx = 0; idx < kTileLoads; ++idx) dma_one(lds_a1, lds_b1, min(BK, last_k0), idx);

  // One K-tile in buffer CUR: this wave's groups, the last one closing the
  // tile (wait for the next tile, barrier, then the loads of tile t + 2 into
  // the buffer just finished).
  auto step = [&](int t, auto cur_tag) {
    constexpr int kCur = decltype(cur_tag)::value;
    float* la = kCur ? lds_a1 : lds_a0;
    float* lb = kCur ? lds_b1 : lds_b0;
    float* la_next = kCur ? lds_a0 : lds_a1;
    float* lb_next = kCur ? lds_b0 : lds_b1;
    const int k_next2 = min((t + 2) * BK, last_k0);
#pragma unroll
    for (int qi = 0; qi < C_::kMyGroups; ++qi) {
      Frag& fc = (qi & 1) ? f1 : f0;
      Frag& fn = (qi & 1) ? f0 : f1;
      if (qi < C_::kMyGroups - 1) {
#pragma unroll
        for (int i = 0; i < kMfmaPerGroup; ++i) {
          mfma_one(fc, i);
          if (i < kReadsPerGroup) read_one(fn, la, lb, qi + 1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kHalf; ++i) mfma_one(fc, i);
        __builtin_amdgcn_sched_barrier(0);
        // the next tile is in LDS and every wave is done with this one
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
          mfma_one(fc, kHalf + i);
#pragma unroll
          for (int r = 0; r < kReadsPer; ++r)
            if (i * kReadsPer + r < kReadsPerGroup)
              read_one(fn, la_next, lb_next, 0, i * kReadsPer + r);
#pragma unroll
          for (int l = 0; l < kLoadsPer; ++l)
            if (i * kLoadsPer + l < kTileLoads) dma_one(la, lb, k_next2, i * kLoadsPer + l);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  for (int t = 0; t < ktiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ktiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  // no load into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (kDual) acc[0][0] += acc_odd;
}

template <int BM, int BN, int BK, int WM, int WN, int KS>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * KS * 64)
    __attribute__((amdgpu_waves_per_eu(KS)))
    mfma_dma_ks_kernel(Problem p, int tiles_m, int tiles_n, int kchunk, float* part, Epilogue ep) {
  using C_ = KsCfg<BM, BN, BK, WM, WN, KS>;
  __shared__ __attribute__((aligned(16))) float lds_a0[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_a1[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b0[C_::kLdsB];
  __shared__ __attribute__((aligned(16))) float lds_b1[C_::kLdsB];
  __shared__ float red[C_::kRed];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  select_batch(p);

  // workgroup -> (K slice, tile), as in the other tiled kernels
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
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global sources of this lane's chunk in each load (all waves) -------
  const float* a_src[C_::kVecA];
#pragma unroll
  for (int v = 0; v < C_::kVecA; ++v) {
    const int chunk = (v * C_::kWaves + wave) * 64 + lane;
    const int m = chunk / C_::kChunksA, cp = chunk % C_::kChunksA;
    const int c = cp ^ swz_a<C_::kChunksA>(m);
    const int gr = m0 + m;
    a_src[v] = p.A + (int64_t)(gr < M ? gr : 0) * p.lda + 4 * c;
  }
  const float* b_src[C_::kVecB];
#pragma unroll
  for (int v = 0; v < C_::kVecB; ++v) {
    const int chunk = (v * C_::kWaves + wave) * 64 + lane;
    const int kr = chunk / C_::kChunksB, cp = chunk % C_::kChunksB;
    const int c = cp ^ (swz_b(kr) >> 2);
    const int col = n0 + 4 * c;
    b_src[v] = p.B + (int64_t)kr * p.ldb + (col < N ? col : 0);
  }

  floatx16 acc[C_::kFragM][C_::kFragN];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < C_::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  ks_k_loop<BM, BN, BK, WM, WN, KS>(lds_a0, lds_b0, lds_a1, lds_b1, a_src, b_src, p.ldb, wave,
                                    lane, K / BK, acc);

  // ---- the K shares' partial tiles, added in share order ------------------
  const int kg = wave / C_::kTileWaves, tw = wave % C_::kTileWaves;
  constexpr int kBlockFloats = 16 * 64;
  if (kg > 0) {
#pragma unroll
    for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
      for (int j = 0; j < C_::kFragN; ++j) {
        float* d = red + ((((kg - 1) * C_::kTileWaves + tw) * C_::kFragM + i) * C_::kFragN + j) *
                             kBlockFloats;
#pragma unroll
        for (int r = 0; r < 16; ++r) d[r * 64 + lane] = acc[i][j][r];
      }
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < C_::kFragN; ++j) {
          const float* s = red + ((((g - 1) * C_::kTileWaves + tw) * C_::kFragM + i) *
                                      C_::kFragN + j) * kBlockFloats;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += s[r * 64 + lane];
        }
    // ---- masked epilogue ------------------------------------------------------
    store_blocks<C_::kFragM, C_::kFragN>(acc, p.C, p.ldc, M, N, m0 + (tw % C_::kWavesM) * WM,
                                         n0 + (tw / C_::kWavesM) * WN, lane, part != nullptr, ep);
  }
}

template <int BM, int BN, int BK, int WM, int WN, int KS>
hipError_t launch_dma_ks(const Problem& p, int slices, int kchunk, float* partials,
                         const Epilogue& e, hipStream_t s) {
  using C_ = KsCfg<BM, BN, BK, WM, WN, KS>;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (slices < 1 || tiles * slices > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch ||
      (slices > 1 && p.batch != 1))
    return hipErrorInvalidConfiguration;
  // direct-to-LDS preconditions (every product of a batch: strides multiples of 4)
  if (p.sa % 4 != 0 || p.sb % 4 != 0) return hipErrorInvalidValue;
  if (p.K % BK != 0 || p.lda % 4 != 0 || p.ldb % 4 != 0 || p.N % 4 != 0 ||
      (reinterpret_cast<uintptr_t>(p.A) & 15) != 0 || (reinterpret_cast<uintptr_t>(p.B) & 15) != 0)
    return hipErrorInvalidValue;
  if (slices > 1) {
    if (!partials || kchunk <= 0 || kchunk % BK != 0 ||
        (int64_t)(slices - 1) * kchunk >= p.K || (int64_t)slices * kchunk < p.K)
      return hipErrorInvalidValue;
  }
  Problem pp = p;
  int tm = tiles_m, tn = tiles_n, kc = kchunk;
  float* part = slices > 1 ? partials : nullptr;
  Epilogue ee = e;
  void* args[] = {&pp, &tm, &tn, &kc, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_dma_ks_kernel<BM, BN, BK, WM, WN, KS>),
      dim3((unsigned)(tiles * slices), 1, (unsigned)p.batch), dim3(C_::kThreads), args, 0, s);
  if (err != hipSuccess || slices == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: mfma_<BM>x<BN>x<BK>_w<WM>x<WN>_kw<KS>_d6_vec (KS waves per wave tile).
#define GEMMF32_MFMA_DMA_KS(BM, BN, BK, WM, WN, KS)                                          \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_kw" #KS "_d6_vec", BM, BN, BK, WM, WN, true, \
   true, true, &launch_dma_ks<BM, BN, BK, WM, WN, KS>}

// Tuning sweeps compare these with the other tiles (GEMM_F32_SWEEP builds).
#if GEMM_F32_SWEEP
const MfmaVariant kDmaKsVariants[] = {
    GEMMF32_MFMA_DMA_KS(64, 64, 32, 32, 32, 2),
    GEMMF32_MFMA_DMA_KS(64, 64, 64, 32, 32, 2),
    GEMMF32_MFMA_DMA_KS(64, 64, 64, 32, 32, 4),
    GEMMF32_MFMA_DMA_KS(128, 64, 32, 64, 32, 2),
    GEMMF32_MFMA_DMA_KS(64, 128, 32, 32, 64, 2),
    GEMMF32_MFMA_DMA_KS(128, 128, 32, 64, 64, 2),
};
constexpr int kDmaKsCount = (int)(sizeof(kDmaKsVariants) / sizeof(kDmaKsVariants[0]));
#else
const MfmaVariant* const kDmaKsVariants = nullptr;
constexpr int kDmaKsCount = 0;
#endif

}  // namespace

int mfma_dma_ks_variant_count() { return kDmaKsCount; }
const MfmaVariant& mfma_dma_ks_variant(int i) { return kDmaKsVariants[i]; }

}  // namespace gemmf32
