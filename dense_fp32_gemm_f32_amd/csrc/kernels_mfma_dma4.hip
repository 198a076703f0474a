// Macro-tiled fp32 GEMM on the CDNA4 matrix cores with direct global -> LDS
// copies of single floats, for operands of any pitch and alignment (gfx950).
//
// The direct-to-LDS kernel (kernels_mfma_dma.hip) moves 16 bytes per lane
// with global_load_lds_dwordx4, which needs 16-byte aligned rows, K a multiple
// of the K-tile and N a multiple of 4; otherwise the tiles are staged through
// registers and written to LDS by the waves (kernels_mfma.hip), whose LDS
// writes compete with the fragment reads.  Here every copy is a
// global_load_lds_dword: lane l moves one float (4-byte alignment only) to
// LDS at the wave's address + 4 l, so a copy fills 64 consecutive floats of
// the tile's LDS image -- two rows of an A tile with BK = 32, a third of a B
// row with BN = 192 -- and each lane fetches whichever float the swizzled
// layout puts there.  Tile, LDS layout, swizzles, fragments, MFMA order and
// schedule are those of the 16-byte kernel; a K-tile takes four times as many
// copy instructions.
//
// Addresses: each copy is a 32-bit per-lane byte offset from a wave-uniform
// 64-bit base (A + (m0 lda + k) 4, B + (k ldb + n0) 4 for the tile's first k),
// so the offsets are computed once and only the scalar base advances with k.
// Rows of A past M and columns of B past N read row M - 1 / column N - 1 and
// only reach rows and columns of C that are not stored.
//
// K: tile t covers k = BK t - pad ... BK t - pad + BK - 1 with pad = (BK -
// K % BK) % BK, so every tile but the first is whole.  The first is staged
// through registers with zeros for k < 0; it is the only tile read with guards,
// and no copy ever reads before the start of a row.  Needs K >= 2 BK, one
// product per K (no K split).
#include <cstdint>
#include <type_traits>

#include "gemm_f32_internal.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

// One global_load_lds_dword: lane l copies the float at base + off_bytes into
// LDS at lds_wave + 4 l.  The LDS address comes from M0 (saved and restored
// around it); written as inline assembly, as the 16-byte copy is, so that the
// kernel alone decides which waits reads of a buffer need.
__device__ __forceinline__ void load_lds4(uint32_t off_bytes, const void* base, float* lds_wave) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) float*)lds_wave));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off_bytes), "s"(base), "s"(lds_addr)
      : "memory");
}

template <int BM, int BN, int BK, int WM, int WN>
struct D4Cfg {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  static constexpr int kWaves = C_::kThreads / 64;
  static constexpr int kSegA = BM * BK / 64 / kWaves;   // 64-float copies of A per wave
  static constexpr int kSegB = BK * BN / 64 / kWaves;   // and of B
  static_assert((BM * BK / 64) % kWaves == 0 && (BK * BN / 64) % kWaves == 0,
                "the 64-float copies divide evenly over the waves");
  static_assert(BK <= 64 && 64 % BK == 0 && BN % 64 == 0,
                "whole rows per copy of A, whole copies per row of B");
};

template <int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void d4_k_loop(float* lds_a0, float* lds_b0, float* lds_a1, float* lds_b1,
                                          const char* a_base, const char* b_base,
                                          int64_t a_step, int64_t b_step,
                                          const uint32_t (&a_off)[D4Cfg<BM, BN, BK, WM, WN>::kSegA],
                                          const uint32_t (&b_off)[D4Cfg<BM, BN, BK, WM, WN>::kSegB],
                                          int wave, int lane, int ktiles,
                                          floatx16 (&acc)[WM / 32][WN / 32]) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  using D_ = D4Cfg<BM, BN, BK, WM, WN>;
  constexpr int kWaves = D_::kWaves;
  constexpr int kTileLoads = D_::kSegA + D_::kSegB;
  // the bases of K-tile t (1 <= t < ktiles): a_base + t a_step, b_base + t
  // b_step, made wave-uniform scalars once per tile
  struct Bases {
    const char* a;
    const char* b;
  };
  auto uniform = [](const char* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
  };
  auto bases = [&](int t) {
    return Bases{uniform(a_base + (int64_t)t * a_step), uniform(b_base + (int64_t)t * b_step)};
  };
  // copy idx of a tile into the LDS buffer (la, lb)
  auto dma_one = [&](float* la, float* lb, const Bases& bs, int idx) {
    if (idx < D_::kSegA) {
      load_lds4(a_off[idx], bs.a, la + (idx * kWaves + wave) * 64);
    } else {
      const int v = idx - D_::kSegA;
      load_lds4(b_off[v], bs.b, lb + (v * kWaves + wave) * 64);
    }
  };

  const int wmi = wave % C_::kWavesM, wni = wave / C_::kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  int a_frag[C_::kFragM][BK / 8];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i) {
    const int row = wmi * WM + 32 * i + lr;
#pragma unroll
    for (int q = 0; q < BK / 8; ++q)
      a_frag[i][q] = row * BK + 4 * ((2 * q + lk) ^ swz_a<C_::kChunksA>(row));
  }
  int b_frag[C_::kFragN];
#pragma unroll
  for (int j = 0; j < C_::kFragN; ++j) b_frag[j] = (wni * WN + 32 * j + lr) ^ (lk << 5);

  struct Frag {
    float4 a[C_::kFragM];
    float b[4][C_::kFragN];
  };
  auto read_one = [&](Frag& f, const float* la, const float* lb, int q, int idx) {
    if (idx < C_::kFragM) {
      f.a[idx] = *reinterpret_cast<const float4*>(&la[a_frag[idx][q]]);
    } else {
      const int j = (idx - C_::kFragM) / 2, s0 = 2 * ((idx - C_::kFragM) % 2);
      f.b[s0][j] = lb[(8 * q + 4 * lk + s0) * BN + b_frag[j]];
      f.b[s0 + 1][j] = lb[(8 * q + 4 * lk + s0 + 1) * BN + b_frag[j]];
    }
  };
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

  // Tile 0 is in buffer 0 (the caller staged it); tile 1 goes to buffer 1.
  // Every step has the same branch-free shape: the copies of a tile past the
  // end re-read the last tile into the buffer that is no longer needed, and
  // the last step reads fragments it will not use.
  const int last = ktiles - 1;   // >= 1
  Frag f0, f1;
#pragma unroll
  for (int idx = 0; idx < kReadsPerGroup; ++idx) read_one(f0, lds_a0, lds_b0, 0, idx);
  {
    const Bases b1 = bases(1);
#pragma unroll
    for (int idx = 0; idx < kTileLoads; ++idx) dma_one(lds_a1, lds_b1, b1, idx);
  }

  auto step = [&](int t, auto cur_tag) {
    constexpr int kCur = decltype(cur_tag)::value;
    float* la = kCur ? lds_a1 : lds_a0;
    float* lb = kCur ? lds_b1 : lds_b0;
    float* la_next = kCur ? lds_a0 : lds_a1;
    float* lb_next = kCur ? lds_b0 : lds_b1;
    const Bases bn2 = bases(min(t + 2, last));
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
            if (i * kLoadsPer + l < kTileLoads) dma_one(la, lb, bn2, i * kLoadsPer + l);
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
}

template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_d4_kernel(Problem p, int tiles_m, int tiles_n, Epilogue ep) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  using D_ = D4Cfg<BM, BN, BK, WM, WN>;
  constexpr int kWaves = D_::kWaves;
  __shared__ __attribute__((aligned(16))) float lds_a0[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_a1[C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b0[C_::kLdsB];
  __shared__ __attribute__((aligned(16))) float lds_b1[C_::kLdsB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  select_batch(p);

  int lin = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(lin, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int pad = (BK - K % BK) % BK;
  const int ktiles = (K + pad) / BK;

  // ---- each lane's float in each copy: tile row / column and k ------------
  // A copy v of this wave fills LDS floats [64 (v kWaves + wave), + 64): row
  // f / BK, physical position f % BK, i.e. logical chunk pos / 4 ^ swz_a(row).
  uint32_t a_off[D_::kSegA];
  int a_row[D_::kSegA], a_k[D_::kSegA];
#pragma unroll
  for (int v = 0; v < D_::kSegA; ++v) {
    const int f = (v * kWaves + wave) * 64 + lane;
    const int row = f / BK, pos = f % BK;
    const int k = 4 * ((pos >> 2) ^ swz_a<C_::kChunksA>(row)) + (pos & 3);
    const int gr = min(m0 + row, M - 1) - m0;   // rows past M read row M - 1
    a_row[v] = gr;
    a_k[v] = k;
    a_off[v] = (uint32_t)(((int64_t)gr * p.lda + k) * 4);
  }
  // B copy v fills floats [64 (v kWaves + wave), + 64) of the [k][n] image:
  // row f / BN, physical column f % BN, logical column that ^ swz_b(row).
  uint32_t b_off[D_::kSegB];
  int b_row[D_::kSegB], b_col[D_::kSegB];
#pragma unroll
  for (int v = 0; v < D_::kSegB; ++v) {
    const int f = (v * kWaves + wave) * 64 + lane;
    const int kr = f / BN, np = f % BN;
    const int gc = min(n0 + (np ^ swz_b(kr)), N - 1) - n0;   // columns past N read column N - 1
    b_row[v] = kr;
    b_col[v] = gc;
    b_off[v] = (uint32_t)(((int64_t)kr * p.ldb + gc) * 4);
  }

  // ---- tile 0 through registers: k < 0 (the pad) reads as zero ------------
  {
    const float* a_t0 = p.A + (int64_t)m0 * p.lda - pad;
    const float* b_t0 = p.B + n0 - (int64_t)pad * p.ldb;
#pragma unroll
    for (int v = 0; v < D_::kSegA; ++v) {
      const int kk = a_k[v] - pad;   // global k of this float in tile 0
      lds_a0[(v * kWaves + wave) * 64 + lane] =
          kk >= 0 ? a_t0[(int64_t)a_row[v] * p.lda + a_k[v]] : 0.f;
    }
#pragma unroll
    for (int v = 0; v < D_::kSegB; ++v) {
      const int kk = b_row[v] - pad;
      lds_b0[(v * kWaves + wave) * 64 + lane] =
          kk >= 0 ? b_t0[(int64_t)b_row[v] * p.ldb + b_col[v]] : 0.f;
    }
  }
  __syncthreads();

  floatx16 acc[C_::kFragM][C_::kFragN];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < C_::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // tile t >= 1 starts at k = BK t - pad >= 0
  const char* a_base = reinterpret_cast<const char*>(p.A + (int64_t)m0 * p.lda - pad);
  const char* b_base = reinterpret_cast<const char*>(p.B + n0 - (int64_t)pad * p.ldb);
  d4_k_loop<BM, BN, BK, WM, WN>(lds_a0, lds_b0, lds_a1, lds_b1, a_base, b_base,
                                (int64_t)BK * 4, (int64_t)BK * p.ldb * 4, a_off, b_off, wave,
                                lane, ktiles, acc);

  store_blocks<C_::kFragM, C_::kFragN>(acc, p.C, p.ldc, M, N, m0 + (wave % C_::kWavesM) * WM,
                                       n0 + (wave / C_::kWavesM) * WN, lane, false, ep);
}

template <int BM, int BN, int BK, int WM, int WN, int kMinWaves>
hipError_t launch_d4(const Problem& p, int slices, int kchunk, float* partials, const Epilogue& e,
                     hipStream_t s) {
  (void)kchunk;
  (void)partials;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (slices != 1 || tiles > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch)
    return hipErrorInvalidConfiguration;
  // whole tiles after the first; 32-bit lane offsets within a tile
  if (p.K < 2 * BK || (int64_t)BM * p.lda * 4 >= (INT64_C(1) << 31) ||
      (int64_t)BK * p.ldb * 4 >= (INT64_C(1) << 31))
    return hipErrorInvalidValue;
  Problem pp = p;
  int tm = tiles_m, tn = tiles_n;
  Epilogue ee = e;
  void* args[] = {&pp, &tm, &tn, &ee};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_d4_kernel<BM, BN, BK, WM, WN, kMinWaves>),
      dim3((unsigned)tiles, 1, (unsigned)p.batch), dim3(Cfg<BM, BN, BK, WM, WN>::kThreads), args,
      0, s);
}

// Name: mfma_<BM>x<BN>x<BK>_w<WM>x<WN>_d4_vec (single-float direct copies).
#define GEMMF32_MFMA_D4(BM, BN, BK, WM, WN, MW)                                           \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_d4_vec", BM, BN, BK, WM, WN, true, true, \
   false, &launch_d4<BM, BN, BK, WM, WN, MW>, true}

// The default build holds the tiles the tuning table can pick; a build with
// GEMM_F32_SWEEP also holds the ones tuning sweeps compared them with.
const MfmaVariant kD4Variants[] = {
    // 64 x 64: the fastest tile with these copies at every unaligned shape
    // tried, from 767 x 769 x 771 to 4096 x 4097 x 4096; BK = 16 (16 KiB of
    // LDS, up to 7 waves per SIMD) for the larger grids (2047 x 3001 x 1531:
    // 150.3 against 152.9 us; 4095^3: 1030 against 1052 us), BK = 32 below
    // (1023 x 1025 x 1027: 42.6 against 43.8 us)
    GEMMF32_MFMA_D4(64, 64, 32, 32, 32, 4),
    GEMMF32_MFMA_D4(64, 64, 16, 32, 32, 6),
#if GEMM_F32_SWEEP
    GEMMF32_MFMA_D4(128, 192, 32, 32, 96, 2),
    GEMMF32_MFMA_D4(192, 128, 32, 96, 32, 2),
    GEMMF32_MFMA_D4(128, 128, 32, 64, 32, 2),
    GEMMF32_MFMA_D4(128, 128, 32, 64, 64, 2),
    GEMMF32_MFMA_D4(128, 64, 32, 64, 32, 3),
    GEMMF32_MFMA_D4(64, 128, 32, 32, 64, 3),
    GEMMF32_MFMA_D4(64, 64, 64, 32, 32, 4),
#endif
};

}  // namespace

int mfma_d4_variant_count() { return (int)(sizeof(kD4Variants) / sizeof(kD4Variants[0])); }
const MfmaVariant& mfma_d4_variant(int i) { return kD4Variants[i]; }

}  // namespace gemmf32
