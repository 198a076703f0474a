// Macro-tiled fp32 GEMM on the CDNA4 matrix cores with direct global -> LDS
// loads (gfx950).
//
// Same tiles, LDS layout, fragments and MFMA order as the kernel in
// kernels_mfma.hip, but the tiles of A and B travel from global memory into
// LDS with global_load_lds_dwordx4: a wave's 64 lanes each move 16 bytes, and
// lane l's bytes land at the wave's LDS address + 16 l.  So the LDS layout is
// fixed by which global chunk each lane fetches: lane l of load v of wave w
// fetches the chunk that the swizzled layout puts at chunk (v * waves + w) *
// 64 + l.  No staging registers, no LDS write instructions.
//
// Two LDS buffers: the loads of K-tile t + 2 go into the buffer that tile t has
// just finished with, right after the barrier that ends tile t; they are
// waited for at the barrier that ends tile t + 1.  Each memory instruction
// is issued right after an MFMA, as in the SCHED 5 loop of the other kernel.
//
// Preconditions (checked by the dispatcher): A and B 16-byte aligned, lda,
// ldb and N multiples of 4, K a multiple of BK.  Rows of A past M and columns
// of B past N are read at clamped addresses and only reach rows and columns
// of C that are not stored.
#include <cstdint>
#include <type_traits>

#include "gemm_f32_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"
#include "stamps.h"

namespace gemmf32 {
namespace {

using namespace mfma;

// The K loop.
template <int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void dma_k_loop(float* lds_a0, float* lds_b0, float* lds_a1, float* lds_b1,
                                           const float* const (&a_src)[Cfg<BM, BN, BK, WM, WN>::kVecA],
                                           const float* const (&b_src)[Cfg<BM, BN, BK, WM, WN>::kVecB],
                                           int64_t ldb, int wave, int lane, int ktiles,
                                           floatx16 (&acc)[WM / 32][WN / 32]) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  constexpr int kWaves = C_::kThreads / 64;
  constexpr int kTileLoads = C_::kVecA + C_::kVecB;
  // load idx of K-tile k0 into the LDS buffer (la, lb)
  auto dma_one = [&](float* la, float* lb, int k0, int idx) {
    if (idx < C_::kVecA) {
      load_lds16(a_src[idx] + k0, la + (idx * kWaves + wave) * 256);
    } else {
      const int v = idx - C_::kVecA;
      load_lds16(b_src[v] + (int64_t)k0 * ldb, lb + (v * kWaves + wave) * 256);
    }
  };

  // ---- fragments and MFMAs (layout as in the register-staged kernel) -----
  const int wmi = wave % C_::kWavesM, wni = wave / C_::kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  int a_off[C_::kFragM][BK / 8];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i) {
    const int row = wmi * WM + 32 * i + lr;
#pragma unroll
    for (int q = 0; q < BK / 8; ++q)
      a_off[i][q] = row * BK + 4 * ((2 * q + lk) ^ swz_a<C_::kChunksA>(row));
  }
  int b_off[C_::kFragN];
#pragma unroll
  for (int j = 0; j < C_::kFragN; ++j) b_off[j] = (wni * WN + 32 * j + lr) ^ (lk << 5);

  struct Frag {
    float4 a[C_::kFragM];
    float b[4][C_::kFragN];
  };
  auto read_one = [&](Frag& f, const float* la, const float* lb, int q, int idx) {
    if (idx < C_::kFragM) {
      f.a[idx] = *reinterpret_cast<const float4*>(&la[a_off[idx][q]]);
    } else {
      const int j = (idx - C_::kFragM) / 2, s0 = 2 * ((idx - C_::kFragM) % 2);
      f.b[s0][j] = lb[(8 * q + 4 * lk + s0) * BN + b_off[j]];
      f.b[s0 + 1][j] = lb[(8 * q + 4 * lk + s0 + 1) * BN + b_off[j]];
    }
  };
  // A wave tile of one 32 x 32 block would chain every MFMA on one
  // accumulator; there the odd k-steps go to a second accumulator, added to
  // the first after the loop (a fixed order: even steps + odd steps).
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

  constexpr int kGroups = BK / 8;
  static_assert(kGroups % 2 == 0, "fragment ping-pong needs an even group count");
  constexpr int kMfmaPerGroup = 4 * C_::kFragM * C_::kFragN;
  constexpr int kHalf = kMfmaPerGroup / 2;
  constexpr int kReadsPerGroup = C_::kFragM + 2 * C_::kFragN;
  constexpr int kReadsPer = (kReadsPerGroup + kHalf - 1) / kHalf;
  constexpr int kLoadsPer = (kTileLoads + kHalf - 1) / kHalf;

  // Every step below has the same branch-free shape: the loads of a tile past
  // the end re-read the last tile into the buffer that is no longer needed,
  // and the last step reads fragments it will not use.
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

  // One K-tile in buffer CUR.
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
        // one fragment read after each MFMA
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

// One workgroup's tile.  With kStamp (the instrumented kernel of the sweep
// build), thread 0 also writes six 64-bit words to stamps[6 w ..] for
// workgroup w: the constant 100 MHz counter (s_memrealtime) at the start,
// after the K loop and after the C stores, then the shader cycle counter
// (s_memtime) at the same three points.  Barriers before the second and third
// readings make them cover every wave, and the third waits for the stores.
template <int BM, int BN, int BK, int WM, int WN, bool kStamp>
__device__ __forceinline__ void dma_tile(float* lds_a0, float* lds_a1, float* lds_b0,
                                         float* lds_b1, Problem p, int tiles_m, int tiles_n,
                                         int kchunk, float* part, const Epilogue& ep,
                                         unsigned long long* stamps) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  constexpr int kWaves = C_::kThreads / 64;
  unsigned long long rt[3] = {}, mt[3] = {};
  if constexpr (kStamp) {
    rt[0] = __builtin_amdgcn_s_memrealtime();
    mt[0] = __builtin_amdgcn_s_memtime();
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  select_batch(p);

  // workgroup -> (K slice, tile), as in the register-staged kernel
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

  // ---- global sources of this lane's chunk in each load ------------------
  const float* a_src[C_::kVecA];
#pragma unroll
  for (int v = 0; v < C_::kVecA; ++v) {
    const int chunk = (v * kWaves + wave) * 64 + lane;
    const int m = chunk / C_::kChunksA, cp = chunk % C_::kChunksA;
    const int c = cp ^ swz_a<C_::kChunksA>(m);
    const int gr = m0 + m;
    a_src[v] = p.A + (int64_t)(gr < M ? gr : 0) * p.lda + 4 * c;
  }
  const float* b_src[C_::kVecB];
#pragma unroll
  for (int v = 0; v < C_::kVecB; ++v) {
    const int chunk = (v * kWaves + wave) * 64 + lane;
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

  dma_k_loop<BM, BN, BK, WM, WN>(lds_a0, lds_b0, lds_a1, lds_b1, a_src, b_src, p.ldb, wave, lane,
                                 K / BK, acc);
  if constexpr (kStamp) {
    __syncthreads();
    rt[1] = __builtin_amdgcn_s_memrealtime();
    mt[1] = __builtin_amdgcn_s_memtime();
  }

  // ---- masked epilogue ------------------------------------------------------
  store_blocks<C_::kFragM, C_::kFragN>(acc, p.C, p.ldc, M, N, m0 + (wave % C_::kWavesM) * WM,
                                       n0 + (wave / C_::kWavesM) * WN, lane, part != nullptr,
                                       ep);
  if constexpr (kStamp) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    rt[2] = __builtin_amdgcn_s_memrealtime();
    mt[2] = __builtin_amdgcn_s_memtime();
    if (tid == 0) {
      unsigned long long* w = stamps + 6 * (size_t)blockIdx.x;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        w[i] = rt[i];
        w[3 + i] = mt[i];
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_dma_kernel(Problem p, int tiles_m, int tiles_n, int kchunk, float* part, Epilogue ep) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  __shared__ __attribute__((aligned(16))) float lds_a0[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_a1[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b0[C_::kLdsB];
  __shared__ __attribute__((aligned(16))) float lds_b1[C_::kLdsB];
  dma_tile<BM, BN, BK, WM, WN, false>(lds_a0, lds_a1, lds_b0, lds_b1, p, tiles_m, tiles_n, kchunk,
                                      part, ep, nullptr);
}

template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
hipError_t launch_dma(const Problem& p, int slices, int kchunk, float* partials, const Epilogue& e,
                      hipStream_t s) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
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
      reinterpret_cast<const void*>(&mfma_dma_kernel<BM, BN, BK, WM, WN, kMinWaves>),
      dim3((unsigned)(tiles * slices), 1, (unsigned)p.batch), dim3(C_::kThreads), args, 0, s);
  if (err != hipSuccess || slices == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

#if GEMM_F32_SWEEP
// The same tile with per-workgroup timestamps (whole K, one product).
template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_dma_stamp_kernel(Problem p, int tiles_m, int tiles_n, Epilogue ep,
                          unsigned long long* stamps) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  __shared__ __attribute__((aligned(16))) float lds_a0[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_a1[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b0[C_::kLdsB];
  __shared__ __attribute__((aligned(16))) float lds_b1[C_::kLdsB];
  dma_tile<BM, BN, BK, WM, WN, true>(lds_a0, lds_a1, lds_b0, lds_b1, p, tiles_m, tiles_n, p.K,
                                     nullptr, ep, stamps);
}

template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
hipError_t launch_dma_stamp(const Problem& p, const Epilogue& e, unsigned long long* stamps,
                            int64_t words, hipStream_t s) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles > 0x7fffffff || p.batch != 1 || !stamps || words < 6 * tiles)
    return hipErrorInvalidConfiguration;
  if (p.K % BK != 0 || p.lda % 4 != 0 || p.ldb % 4 != 0 || p.N % 4 != 0 ||
      (reinterpret_cast<uintptr_t>(p.A) & 15) != 0 || (reinterpret_cast<uintptr_t>(p.B) & 15) != 0)
    return hipErrorInvalidValue;
  Problem pp = p;
  int tm = tiles_m, tn = tiles_n;
  Epilogue ee = e;
  unsigned long long* st = stamps;
  void* args[] = {&pp, &tm, &tn, &ee, &st};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_dma_stamp_kernel<BM, BN, BK, WM, WN, kMinWaves>),
      dim3((unsigned)tiles), dim3(C_::kThreads), args, 0, s);
}
#endif

// The tiles: the default build holds the ones the tuning table can pick; a
// build with GEMM_F32_SWEEP also holds the ones tuning sweeps compared them
// with.
#define GEMMF32_DMA_TILES(X) \
  X(256, 256, 32, 64, 128, 1) \
  X(128, 256, 16, 64, 128, 2) \
  X(128, 192, 32, 32, 96, 2)  \
  X(192, 128, 32, 96, 32, 2)  \
  X(128, 128, 32, 64, 32, 2)  \
  X(128, 128, 16, 64, 64, 3)  \
  X(64, 64, 32, 32, 32, 4)
#define GEMMF32_DMA_SWEEP_TILES(X) \
  X(256, 128, 16, 128, 64, 2)      \
  X(256, 128, 32, 128, 64, 1)      \
  X(128, 128, 32, 64, 64, 2)       \
  X(128, 128, 64, 64, 64, 1)       \
  X(128, 64, 32, 64, 32, 3)        \
  X(128, 64, 64, 64, 32, 2)        \
  X(64, 64, 64, 32, 32, 2)         \
  X(256, 256, 16, 128, 64, 1)      \
  X(256, 256, 16, 64, 128, 1)      \
  X(256, 256, 32, 128, 64, 1)

#define GEMMF32_MFMA_DMA(BM, BN, BK, WM, WN, MW)                                          \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d6_vec", BM, BN, BK, WM, WN, true, true, \
   true, &launch_dma<BM, BN, BK, WM, WN, MW>},

const MfmaVariant kDmaVariants[] = {
    GEMMF32_DMA_TILES(GEMMF32_MFMA_DMA)
#if GEMM_F32_SWEEP
    GEMMF32_DMA_SWEEP_TILES(GEMMF32_MFMA_DMA)
#endif
};

#if GEMM_F32_SWEEP
using StampLaunch = hipError_t (*)(const Problem&, const Epilogue&, unsigned long long*, int64_t,
                                   hipStream_t);
#define GEMMF32_DMA_STAMP(BM, BN, BK, WM, WN, MW) &launch_dma_stamp<BM, BN, BK, WM, WN, MW>,
// in the order of kDmaVariants
const StampLaunch kDmaStamped[] = {GEMMF32_DMA_TILES(GEMMF32_DMA_STAMP)
                                       GEMMF32_DMA_SWEEP_TILES(GEMMF32_DMA_STAMP)};
static_assert(sizeof(kDmaStamped) / sizeof(kDmaStamped[0]) ==
                  sizeof(kDmaVariants) / sizeof(kDmaVariants[0]),
              "one instrumented launch per tile");
#endif

}  // namespace

int mfma_dma_variant_count() { return (int)(sizeof(kDmaVariants) / sizeof(kDmaVariants[0])); }
#if GEMM_F32_SWEEP
hipError_t launch_dma_stamped(int i, const Problem& p, const Epilogue& e,
                              unsigned long long* stamps, int64_t words, hipStream_t s) {
  if (i < 0 || i >= mfma_dma_variant_count()) return hipErrorInvalidValue;
  return kDmaStamped[i](p, e, stamps, words, s);
}
#endif
const MfmaVariant& mfma_dma_variant(int i) { return kDmaVariants[i]; }

}  // namespace gemmf32
