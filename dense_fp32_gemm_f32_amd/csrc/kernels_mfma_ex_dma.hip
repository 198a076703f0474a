// Extended operation C = act(alpha * op(A) op(B) + beta * C + bias) with
// direct global -> LDS loads (gfx950), for operands stored either way.
//
// The MFMA operands of v_mfma_f32_32x32x2_f32 are symmetric (lane l of the A
// operand holds A[l % 32][k-slot l / 32], lane l of the B operand B[k-slot
// l / 32][l % 32]), so one operand description serves A (rows = m) and B
// (rows = n) in either storage:
//   KC  ("k contiguous"): element (r, k) at X[r * ld + k]   (A as is, B^T)
//   RC  ("r contiguous"): element (r, k) at X[k * ld + r]   (A^T, B as is)
// In LDS a KC operand is [r][k] with its 16-byte chunks swizzled by row and is
// read with 128-bit fragment reads (the k-slot permutation of the plain
// kernels); an RC operand is [k][r] with r XORed by 32 on bit 2 of k and is
// read with 32-bit fragment reads.
//
// The tiles travel with global_load_lds_dwordx4 as in kernels_mfma_dma.hip:
// lane l of a wave's load lands at the wave's LDS address + 16 l, so each lane
// fetches the global chunk that the swizzled layout puts at its position.  Two
// LDS buffers, one barrier per K-tile, loads of K-tile t + 2 issued after the
// barrier that ends tile t, each memory instruction right after an MFMA.
//
// Preconditions (checked by the dispatcher and again at launch): A and B
// 16-byte aligned, lda and ldb multiples of 4, K a multiple of BK, and the
// contiguous extent of an RC operand (M for A^T, N for B) a multiple of 4, so
// that a 16-byte chunk lies wholly inside or wholly outside the matrix.  Rows
// (KC) or chunks (RC) past M or N are read at clamped addresses and reach
// only rows and columns of C that are not stored.
#include <cstdint>
#include <type_traits>

#include "gemm_f32_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

// One operand's K-tile: R rows (BM for A, BN for B) by BK, kWaves waves.
template <int R, int BK, int kWaves, bool KC>
struct DmaOperand {
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kChunks = R * BK / 4;            // 16-byte chunks per K-tile
  static constexpr int kLoads = kChunks / kThreads;     // copies per lane
  static constexpr int kLds = R * BK;
  static constexpr int kRowChunks = KC ? BK / 4 : R / 4;
  static_assert(kChunks % kThreads == 0, "chunks divide evenly over the threads");
  static_assert(KC || R % 64 == 0, "the [k][r] swizzle needs 64-wide rows");
  static_assert(!KC || BK / 4 <= 16, "the [r][k] swizzle covers at most 16 chunks");

  const float* src[kLoads];   // this lane's chunk of each copy at K-tile 0

  // LDS position pos (in chunks) holds the chunk of logical (r, k) below.
  __device__ __forceinline__ void init(const float* base, int64_t ld, int r0, int rtot,
                                       int wave, int lane) {
#pragma unroll
    for (int v = 0; v < kLoads; ++v) {
      const int pos = (v * kWaves + wave) * 64 + lane;
      if constexpr (KC) {
        const int r = pos / kRowChunks, cp = pos % kRowChunks;
        const int c = cp ^ swz_a<BK / 4>(r);
        const int gr = r0 + r;
        src[v] = base + (int64_t)(gr < rtot ? gr : 0) * ld + 4 * c;
      } else {
        const int k = pos / kRowChunks, cp = pos % kRowChunks;
        const int c = cp ^ (swz_b(k) >> 2);
        const int gr = r0 + 4 * c;
        src[v] = base + (int64_t)k * ld + (gr < rtot ? gr : 0);
      }
    }
  }
  __device__ __forceinline__ void copy(int v, float* lds, int64_t ld, int k0, int wave) const {
    const int64_t step = KC ? (int64_t)k0 : (int64_t)k0 * ld;
    load_lds16(src[v] + step, lds + (v * kWaves + wave) * 256);
  }

  // Fragment reads of one k group q (8 k) for the wave's blocks starting at
  // tile row wr: KC, one 128-bit read per block (four k-slots); RC, two
  // 32-bit reads per unit, two units per block.
  static constexpr int kUnits(int frags) { return KC ? frags : 2 * frags; }
  template <int kFrag>
  __device__ __forceinline__ static void read(float (&f)[4][kFrag], const float* lds, int wr,
                                              int lr, int lk, int q, int unit) {
    if constexpr (KC) {
      const int row = wr + 32 * unit + lr;
      const float4 x =
          *reinterpret_cast<const float4*>(&lds[row * BK + 4 * ((2 * q + lk) ^ swz_a<BK / 4>(row))]);
      f[0][unit] = x.x;
      f[1][unit] = x.y;
      f[2][unit] = x.z;
      f[3][unit] = x.w;
    } else {
      const int i = unit / 2, s0 = 2 * (unit % 2);
      const int col = (wr + 32 * i + lr) ^ (lk << 5);
      f[s0][i] = lds[(8 * q + 4 * lk + s0) * R + col];
      f[s0 + 1][i] = lds[(8 * q + 4 * lk + s0 + 1) * R + col];
    }
  }
};

template <int BM, int BN, int BK, int WM, int WN, bool A_KC, bool B_KC, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_ex_dma_kernel(Problem p, Epilogue ep, int tiles_m, int tiles_n) {
  constexpr int kWavesM = BM / WM, kWavesN = BN / WN, kWaves = kWavesM * kWavesN;
  constexpr int kFragM = WM / 32, kFragN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % WM == 0 && BN % WN == 0, "32x32 blocks");
  static_assert(BK % 16 == 0, "an even number of 8-k groups per K-tile");
  using OpA = DmaOperand<BM, BK, kWaves, A_KC>;
  using OpB = DmaOperand<BN, BK, kWaves, B_KC>;
  __shared__ __attribute__((aligned(16))) float lds_a0[OpA::kLds];
  __shared__ __attribute__((aligned(16))) float lds_a1[OpA::kLds];
  __shared__ __attribute__((aligned(16))) float lds_b0[OpB::kLds];
  __shared__ __attribute__((aligned(16))) float lds_b1[OpB::kLds];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  select_batch(p);
  const int M = p.M, N = p.N, K = p.K;

  int tm, tn;
  tile_coords(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  OpA opa;
  OpB opb;
  opa.init(p.A, p.lda, m0, M, wave, lane);
  opb.init(p.B, p.ldb, n0, N, wave, lane);
  constexpr int kTileLoads = OpA::kLoads + OpB::kLoads;
  auto copy_one = [&](float* la, float* lb, int k0, int idx) {
    if (idx < OpA::kLoads) {
      opa.copy(idx, la, p.lda, k0, wave);
    } else {
      opb.copy(idx - OpA::kLoads, lb, p.ldb, k0, wave);
    }
  };

  const int wmi = wave % kWavesM, wni = wave / kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  const int wr_a = wmi * WM, wr_b = wni * WN;
  struct Frag {
    float a[4][kFragM];
    float b[4][kFragN];
  };
  constexpr int kUnitsA = OpA::kUnits(kFragM), kUnitsB = OpB::kUnits(kFragN);
  constexpr int kReadsPerGroup = kUnitsA + kUnitsB;
  auto read_one = [&](Frag& f, const float* la, const float* lb, int q, int idx) {
    if (idx < kUnitsA) {
      OpA::template read<kFragM>(f.a, la, wr_a, lr, lk, q, idx);
    } else {
      OpB::template read<kFragN>(f.b, lb, wr_b, lr, lk, q, idx - kUnitsA);
    }
  };

  floatx16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // one 32 x 32 block per wave: the odd k-steps go to a second accumulator,
  // added after the loop (a fixed order: even steps + odd steps)
  constexpr bool kDual = kFragM * kFragN == 1;
  floatx16 acc_odd = {};
  auto mfma_one = [&](const Frag& f, int idx) {
    const int s = idx / (kFragM * kFragN);
    const int i = (idx / kFragN) % kFragM, j = idx % kFragN;
    if constexpr (kDual) {
      if (s & 1) {
        acc_odd = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[s][i], f.b[s][j], acc_odd, 0, 0, 0);
        return;
      }
    }
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[s][i], f.b[s][j], acc[i][j], 0, 0, 0);
  };

  constexpr int kGroups = BK / 8;
  constexpr int kMfmaPerGroup = 4 * kFragM * kFragN;
  constexpr int kHalf = kMfmaPerGroup / 2;
  constexpr int kReadsPer = (kReadsPerGroup + kHalf - 1) / kHalf;
  constexpr int kLoadsPer = (kTileLoads + kHalf - 1) / kHalf;
  static_assert(kReadsPerGroup <= kMfmaPerGroup, "one fragment read after each MFMA");

  // Branch-free steps: the copies of a K-tile past the end re-read the last
  // tile into the buffer no longer needed; the last step reads fragments it
  // does not use.
  const int ktiles = K / BK;
  const int last_k0 = (ktiles - 1) * BK;
  Frag f0, f1;
#pragma unroll
  for (int idx = 0; idx < kTileLoads; ++idx) copy_one(lds_a0, lds_b0, 0, idx);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int idx = 0; idx < kReadsPerGroup; ++idx) read_one(f0, lds_a0, lds_b0, 0, idx);
#pragma unroll
  for (int idx = 0; idx < kTileLoads; ++idx) copy_one(lds_a1, lds_b1, min(BK, last_k0), idx);

  auto step = [&](int t, auto cur_tag) {
    constexpr int kCur = decltype(cur_tag)::value;
    float* la = kCur ? lds_a1 : lds_a0;
    float* lb = kCur ? lds_b1 : lds_b0;
    float* la_next = kCur ? lds_a0 : lds_a1;
    float* lb_next = kCur ? lds_b0 : lds_b1;
    const int k_next2 = min((t + 2) * BK, last_k0);
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      Frag& fc = (q & 1) ? f1 : f0;
      Frag& fn = (q & 1) ? f0 : f1;
      if (q < kGroups - 1) {
#pragma unroll
        for (int i = 0; i < kMfmaPerGroup; ++i) {
          mfma_one(fc, i);
          if (i < kReadsPerGroup) read_one(fn, la, lb, q + 1, i);
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
            if (i * kLoadsPer + l < kTileLoads) copy_one(la, lb, k_next2, i * kLoadsPer + l);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  for (int t = 0; t < ktiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ktiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  // no copy into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (kDual) acc[0][0] += acc_odd;

  // ---- masked epilogue: C = act(alpha * acc + beta * C + bias) ---------------
  store_blocks<kFragM, kFragN>(acc, p.C, p.ldc, M, N, m0 + wr_a, n0 + wr_b, lane, false, ep);
}

template <int BM, int BN, int BK, int WM, int WN, bool A_KC, bool B_KC, int kMinWaves>
hipError_t launch_ex_dma(const Problem& p, const Epilogue& e, hipStream_t s) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch)
    return hipErrorInvalidConfiguration;
  // direct-to-LDS preconditions (every product of a batch: strides multiples of 4)
  if (p.K < BK || p.K % BK != 0 || p.lda % 4 != 0 || p.ldb % 4 != 0 || p.sa % 4 != 0 ||
      p.sb % 4 != 0 || (!A_KC && p.M % 4 != 0) || (!B_KC && p.N % 4 != 0) ||
      (reinterpret_cast<uintptr_t>(p.A) & 15) != 0 || (reinterpret_cast<uintptr_t>(p.B) & 15) != 0)
    return hipErrorInvalidValue;
  Problem pp = p;
  Epilogue ee = e;
  int tm = tiles_m, tn = tiles_n;
  void* args[] = {&pp, &ee, &tm, &tn};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_ex_dma_kernel<BM, BN, BK, WM, WN, A_KC, B_KC, kMinWaves>),
      dim3((unsigned)tiles, 1, (unsigned)p.batch), dim3((BM / WM) * (BN / WN) * 64), args, 0,
      s);
}

// Name: mfmaex_<tile>_d6_<layout>, layout = op(A) op(B) as n (stored as is)
// or t (stored transposed).  A is KC when not transposed; B is KC when
// transposed.
// The default build holds the three layouts with a transposed operand; a
// build with GEMM_F32_SWEEP adds the _nn twins.
#define GEMMF32_MFMA_EX_DMA_T(BM, BN, BK, WM, WN, MW)                                     \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d6_nt", BM, BN, BK, false, true,       \
   &launch_ex_dma<BM, BN, BK, WM, WN, true, true, MW>, true},                              \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d6_tn", BM, BN, BK, true, false,       \
   &launch_ex_dma<BM, BN, BK, WM, WN, false, false, MW>, true},                            \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d6_tt", BM, BN, BK, true, true,        \
   &launch_ex_dma<BM, BN, BK, WM, WN, false, true, MW>, true}
#define GEMMF32_MFMA_EX_DMA_NN(BM, BN, BK, WM, WN, MW)                                    \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d6_nn", BM, BN, BK, false, false,      \
   &launch_ex_dma<BM, BN, BK, WM, WN, true, false, MW>, true}

const MfmaExVariant kExDmaVariants[] = {
    GEMMF32_MFMA_EX_DMA_T(256, 256, 32, 64, 128, 1),
    GEMMF32_MFMA_EX_DMA_T(128, 128, 32, 64, 32, 2),
    GEMMF32_MFMA_EX_DMA_T(64, 64, 32, 32, 32, 4),
#if GEMM_F32_SWEEP
    GEMMF32_MFMA_EX_DMA_NN(256, 256, 32, 64, 128, 1),
    GEMMF32_MFMA_EX_DMA_NN(128, 128, 32, 64, 32, 2),
    GEMMF32_MFMA_EX_DMA_NN(64, 64, 32, 32, 32, 4),
#endif
};

}  // namespace

int mfma_ex_dma_variant_count() {
  return (int)(sizeof(kExDmaVariants) / sizeof(kExDmaVariants[0]));
}
const MfmaExVariant& mfma_ex_dma_variant(int i) { return kExDmaVariants[i]; }

}  // namespace gemmf32
