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
#include <type_traits>

#include "gemm_f32_internal.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

// SCHED 0: the next K-tile is written to LDS after all MFMAs of this one.
// SCHED 1: it is written after the first half of them, so the write, the
//          barrier and the first fragment reads of the next tile overlap the
//          second half.
// SCHED 2: as 1, and the wave runs at raised priority while it issues memory
//          instructions, lowered again for the MFMAs.
// SCHED 3, 4, 5: software pipeline with fragments read one k group ahead
//          and global loads two K-tiles ahead (described at the loop).
template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB, int kMinWaves, int SCHED>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_gemm_kernel(Problem p, int tiles_m, int tiles_n, int kchunk, float* part, Epilogue ep) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  __shared__ __attribute__((aligned(16))) float lds_a[2][C_::kLdsA];
  __shared__ __attribute__((aligned(16))) float lds_b[2][C_::kLdsB];

  const int tid = threadIdx.x;
  select_batch(p);

  // Workgroup -> (K slice, tile).  Consecutive ids of one XCD stay within one
  // slice, so neighbouring tiles of a slice share that XCD's L2.
  const int tiles = tiles_m * tiles_n;
  int lin = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int slice = lin / tiles;
  lin -= slice * tiles;
  if (part) {
    // this slice is the GEMM of A[:, k0:k0+K'] and B[k0:k0+K', :] into its
    // own packed partial buffer
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
  const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);

  // ---- global -> register staging ----------------------------------------
  // A: float4 chunk c of tile row `row` (k = 4c..4c+3).
  // B: float4 chunk of tile row `krow` (n = nc..nc+3).
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
  int b_ncol[C_::kVecB];
#pragma unroll
  for (int v = 0; v < C_::kVecB; ++v) {
    const int e = tid + v * C_::kThreads;
    const int krow = e / C_::kChunksB, nc = (e % C_::kChunksB) * 4;
    b_ncol[v] = n0 + nc;
    b_ptr[v] = p.B + (int64_t)krow * p.ldb + (b_ncol[v] < N ? b_ncol[v] : 0);
  }

  float4 ra[C_::kVecA], rb[C_::kVecB];

  // Interior K-tile of an interior output tile: no masks.
  auto load_tiles_full = [&](int k0) {
#pragma unroll
    for (int v = 0; v < C_::kVecA; ++v) {
      const float* src = a_ptr[v] + k0;
      if (VA) {
        ra[v] = load4(src);
      } else {
        ra[v] = make_float4(src[0], src[1], src[2], src[3]);
      }
    }
#pragma unroll
    for (int v = 0; v < C_::kVecB; ++v) {
      const float* src = b_ptr[v] + (int64_t)k0 * p.ldb;
      if (VB) {
        rb[v] = load4(src);
      } else {
        rb[v] = make_float4(src[0], src[1], src[2], src[3]);
      }
    }
  };
  // Any K-tile: elements outside M x K (A) or K x N (B) become 0.0.
  auto load_tiles_masked = [&](int k0) {
#pragma unroll
    for (int v = 0; v < C_::kVecA; ++v) {
      const int e = tid + v * C_::kThreads;
      const int gk = k0 + (e % C_::kChunksA) * 4;
      const float* src = a_ptr[v] + k0;
      const bool ok = a_row_ok[v];
      if (VA && ok && gk + 3 < K) {
        ra[v] = load4(src);
      } else {
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
      const int nn = b_ncol[v];
      if (VB && kok && nn + 3 < N) {
        rb[v] = load4(src);
      } else {
        rb[v].x = (kok && nn + 0 < N) ? src[0] : 0.f;
        rb[v].y = (kok && nn + 1 < N) ? src[1] : 0.f;
        rb[v].z = (kok && nn + 2 < N) ? src[2] : 0.f;
        rb[v].w = (kok && nn + 3 < N) ? src[3] : 0.f;
      }
    }
  };
  auto load_tiles = [&](int k0) {
    if (full_mn && k0 + BK <= K) {
      load_tiles_full(k0);
    } else {
      load_tiles_masked(k0);
    }
  };

  auto store_tiles = [&](int buf) {
    float* la = lds_a[buf];
    float* lb = lds_b[buf];
#pragma unroll
    for (int v = 0; v < C_::kVecA; ++v) {
      const int e = tid + v * C_::kThreads;
      const int row = e / C_::kChunksA, c = e % C_::kChunksA;
      *reinterpret_cast<float4*>(&la[row * BK + 4 * (c ^ swz_a<C_::kChunksA>(row))]) = ra[v];
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
  // per-lane LDS offsets of the fragments (in floats, within one buffer)
  int a_off[C_::kFragM][BK / 8];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i) {
    const int row = wmi * WM + 32 * i + lr;
#pragma unroll
    for (int q = 0; q < BK / 8; ++q)
      a_off[i][q] = row * BK + 4 * ((2 * q + lk) ^ swz_a<C_::kChunksA>(row));
  }
  // B column of fragment j, swizzled: the k rows a lane reads all have bit 2 == lk
  int b_off[C_::kFragN];
#pragma unroll
  for (int j = 0; j < C_::kFragN; ++j) b_off[j] = (wni * WN + 32 * j + lr) ^ (lk << 5);

  floatx16 acc[C_::kFragM][C_::kFragN];
#pragma unroll
  for (int i = 0; i < C_::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < C_::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMAs of the 8-wide k groups [q0, q1) of LDS buffer `buf`
  auto compute = [&](int buf, int q0, int q1) {
    const float* la = lds_a[buf];
    const float* lb = lds_b[buf];
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      float4 fa[C_::kFragM];
#pragma unroll
      for (int i = 0; i < C_::kFragM; ++i)
        fa[i] = *reinterpret_cast<const float4*>(&la[a_off[i][q]]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int krow = 8 * q + 4 * lk + s;
        float fb[C_::kFragN];
#pragma unroll
        for (int j = 0; j < C_::kFragN; ++j) fb[j] = lb[krow * BN + b_off[j]];
#pragma unroll
        for (int i = 0; i < C_::kFragM; ++i) {
          const float a = s == 0 ? fa[i].x : s == 1 ? fa[i].y : s == 2 ? fa[i].z : fa[i].w;
#pragma unroll
          for (int j = 0; j < C_::kFragN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // Fragments of one 8-wide k group, held in registers one group ahead of
  // the MFMAs that use them (SCHED >= 3).
  struct Frag {
    float4 a[C_::kFragM];
    float b[4][C_::kFragN];
  };
  auto read_frag = [&](Frag& f, int buf, int q) {
    const float* la = lds_a[buf];
    const float* lb = lds_b[buf];
#pragma unroll
    for (int i = 0; i < C_::kFragM; ++i)
      f.a[i] = *reinterpret_cast<const float4*>(&la[a_off[i][q]]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < C_::kFragN; ++j) f.b[s][j] = lb[(8 * q + 4 * lk + s) * BN + b_off[j]];
  };
  // MFMA steps [s0, s1) of a group's fragments
  auto mfma_frag = [&](const Frag& f, int s0, int s1) {
#pragma unroll
    for (int s = s0; s < s1; ++s)
#pragma unroll
      for (int i = 0; i < C_::kFragM; ++i) {
        const float a = s == 0 ? f.a[i].x : s == 1 ? f.a[i].y : s == 2 ? f.a[i].z : f.a[i].w;
#pragma unroll
        for (int j = 0; j < C_::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.b[s][j], acc[i][j], 0, 0, 0);
      }
  };

  // Single instructions of the pipelined loop, so that SCHED 5 can place each
  // one between two MFMAs.  Op `idx` of a group's fragment reads: A block
  // idx (one ds_read_b128), then for B block j the k rows s = 0, 1 and then
  // s = 2, 3 (two b32 reads the compiler pairs into one instruction).
  auto read_one = [&](Frag& f, int buf, int q, int idx) {
    if (idx < C_::kFragM) {
      f.a[idx] = *reinterpret_cast<const float4*>(&lds_a[buf][a_off[idx][q]]);
    } else {
      const int j = (idx - C_::kFragM) / 2, s0 = 2 * ((idx - C_::kFragM) % 2);
      const float* lb = lds_b[buf];
      f.b[s0][j] = lb[(8 * q + 4 * lk + s0) * BN + b_off[j]];
      f.b[s0 + 1][j] = lb[(8 * q + 4 * lk + s0 + 1) * BN + b_off[j]];
    }
  };
  // MFMA number idx of a group, in the order of mfma_frag
  auto mfma_one = [&](const Frag& f, int idx) {
    const int s = idx / (C_::kFragM * C_::kFragN);
    const int i = (idx / C_::kFragN) % C_::kFragM, j = idx % C_::kFragN;
    const float a = s == 0 ? f.a[i].x : s == 1 ? f.a[i].y : s == 2 ? f.a[i].z : f.a[i].w;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.b[s][j], acc[i][j], 0, 0, 0);
  };
  // Global load number idx (A chunks, then B) of a K-tile that lies inside
  // K, for any output tile.  Rows of A past M and columns of B past N are
  // read at the clamped addresses set up above and left unmasked: they only
  // reach rows or columns of C that the epilogue does not store.  NPART: this
  // tile has a B chunk that straddles column N (N % 4 != 0); its B chunks are
  // then read element by element with each column clamped to N - 1, so no
  // read passes the end of a row.
  auto load_one_any = [&](int k0, int idx, auto npart_tag) {
    constexpr bool kNPart = decltype(npart_tag)::value;
    if (idx < C_::kVecA) {
      const float* src = a_ptr[idx] + k0;
      ra[idx] = VA ? load4(src) : make_float4(src[0], src[1], src[2], src[3]);
    } else {
      const int v = idx - C_::kVecA;
      const float* src = b_ptr[v] + (int64_t)k0 * p.ldb;
      if constexpr (kNPart) {
        const float* row = src - (b_ncol[v] < N ? b_ncol[v] : 0);
        const int c = b_ncol[v];
        rb[v] = make_float4(row[min(c, N - 1)], row[min(c + 1, N - 1)], row[min(c + 2, N - 1)],
                            row[min(c + 3, N - 1)]);
      } else {
        rb[v] = VB ? load4(src) : make_float4(src[0], src[1], src[2], src[3]);
      }
    }
  };
  // LDS write number idx of store_tiles
  auto store_one = [&](int buf, int idx) {
    if (idx < C_::kVecA) {
      const int e = tid + idx * C_::kThreads;
      const int row = e / C_::kChunksA, c = e % C_::kChunksA;
      *reinterpret_cast<float4*>(&lds_a[buf][row * BK + 4 * (c ^ swz_a<C_::kChunksA>(row))]) =
          ra[idx];
    } else {
      const int v = idx - C_::kVecA;
      const int e = tid + v * C_::kThreads;
      const int krow = e / C_::kChunksB, nc = (e % C_::kChunksB) * 4;
      *reinterpret_cast<float4*>(&lds_b[buf][krow * BN + (nc ^ swz_b(krow))]) = rb[v];
    }
  };

  // ---- K loop: double-buffered LDS, one barrier per K-tile ---------------
  const int ktiles = (K + BK - 1) / BK;
  constexpr int kGroups = BK / 8;
  if constexpr (SCHED < 3) {
    constexpr int kHalf = SCHED == 0 ? kGroups : (kGroups + 1) / 2;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    for (int t = 0; t < ktiles; ++t) {
      const int cur = t & 1;
      const bool more = t + 1 < ktiles;
      if (SCHED == 2) __builtin_amdgcn_s_setprio(1);
      if (more) load_tiles((t + 1) * BK);
      if (SCHED == 2) __builtin_amdgcn_s_setprio(0);
      compute(cur, 0, kHalf);
      if (SCHED == 2) __builtin_amdgcn_s_setprio(1);
      if (more) store_tiles(cur ^ 1);
      if (SCHED == 2) __builtin_amdgcn_s_setprio(0);
      compute(cur, kHalf, kGroups);
      __syncthreads();
    }
  } else {
    // Software pipeline: the fragments of group q + 1 are read while the
    // MFMAs of group q run; the global loads of tile t + 2 are issued right
    // after the barrier that ends tile t's LDS reads, and written to LDS
    // during tile t + 1 (SCHED 3, 5: with the reads of its last group;
    // SCHED 4: in the middle of the last group's MFMAs, just before the
    // barrier).  sched_barrier keeps the compiler from moving MFMAs across
    // the phases.
    // SCHED 5 runs the K-tiles whose loads all lie inside K in a loop without
    // branches (for edge tiles too, see load_one_any), where the LDS reads, LDS writes and global loads
    // are issued one or two after each MFMA instead of in bursts.
    static_assert(kGroups % 2 == 0, "fragment ping-pong needs an even group count");
    constexpr int kStoreQ = SCHED == 4 ? kGroups - 1 : kGroups - 2;
    constexpr int kMfmaPerGroup = 4 * C_::kFragM * C_::kFragN;
    constexpr int kReadsPerGroup = C_::kFragM + 2 * C_::kFragN;   // b128 A, paired b32 B
    constexpr int kTileLoads = C_::kVecA + C_::kVecB;
    Frag f0, f1;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    read_frag(f0, 0, 0);
    if (ktiles > 1) load_tiles(BK);
    auto step = [&](int t, auto fast_tag, auto npart_tag) {
      constexpr bool kFast = decltype(fast_tag)::value;
      const int cur = t & 1;
      const bool more = kFast || t + 1 < ktiles;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        Frag& fc = (q & 1) ? f1 : f0;
        Frag& fn = (q & 1) ? f0 : f1;
        if constexpr (kFast) {
          // one LDS read / LDS write / global load after each MFMA
          constexpr int kHalf = kMfmaPerGroup / 2;
          if (q < kGroups - 1) {
            constexpr int kWritesPer = (kTileLoads + kMfmaPerGroup - 1) / kMfmaPerGroup;
#pragma unroll
            for (int i = 0; i < kMfmaPerGroup; ++i) {
              mfma_one(fc, i);
              if (i < kReadsPerGroup) read_one(fn, cur, q + 1, i);
              if (q == kStoreQ) {
#pragma unroll
                for (int w = 0; w < kWritesPer; ++w)
                  if (i * kWritesPer + w < kTileLoads) store_one(cur ^ 1, i * kWritesPer + w);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int i = 0; i < kHalf; ++i) mfma_one(fc, i);
            __builtin_amdgcn_sched_barrier(0);
            if (q == kStoreQ) store_tiles(cur ^ 1);
            __syncthreads();
            constexpr int kLoadsPer = (kTileLoads + kHalf - 1) / kHalf;
            constexpr int kReadsPer = (kReadsPerGroup + kHalf - 1) / kHalf;
#pragma unroll
            for (int i = 0; i < kHalf; ++i) {
              mfma_one(fc, kHalf + i);
#pragma unroll
              for (int r = 0; r < kReadsPer; ++r)
                if (i * kReadsPer + r < kReadsPerGroup) read_one(fn, cur ^ 1, 0, i * kReadsPer + r);
#pragma unroll
              for (int l = 0; l < kLoadsPer; ++l)
                if (i * kLoadsPer + l < kTileLoads)
                  load_one_any((t + 2) * BK, i * kLoadsPer + l, npart_tag);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else if (q < kGroups - 1) {
          read_frag(fn, cur, q + 1);
          if (q == kStoreQ && more) store_tiles(cur ^ 1);
          __builtin_amdgcn_sched_barrier(0);
          mfma_frag(fc, 0, 4);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          mfma_frag(fc, 0, 2);
          __builtin_amdgcn_sched_barrier(0);
          if (q == kStoreQ && more) store_tiles(cur ^ 1);
          __syncthreads();
          if (more) {
            read_frag(fn, cur ^ 1, 0);
            if (t + 2 < ktiles) load_tiles((t + 2) * BK);
          }
          __builtin_amdgcn_sched_barrier(0);
          mfma_frag(fc, 2, 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    int t = 0;
    if (SCHED == 5) {
      // K-tiles up to t + 2 inside K: no masks, no branches
      const int kfull = K / BK;
      if (n0 + BN > N && N % 4 != 0) {
        for (; t + 2 < kfull; ++t) step(t, std::true_type{}, std::true_type{});
      } else {
        for (; t + 2 < kfull; ++t) step(t, std::true_type{}, std::false_type{});
      }
    }
    for (; t < ktiles; ++t) step(t, std::false_type{}, std::false_type{});
  }

  // ---- masked epilogue ------------------------------------------------------
  store_blocks<C_::kFragM, C_::kFragN>(acc, p.C, p.ldc, M, N, m0 + (wave % C_::kWavesM) * WM,
                                       n0 + (wave / C_::kWavesM) * WN, lane, part != nullptr,
                                       ep);
}

template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB, int kMinWaves, int SCHED>
hipError_t launch(const Problem& p, int slices, int kchunk, float* partials, const Epilogue& e,
                      hipStream_t s) {
  using C_ = Cfg<BM, BN, BK, WM, WN>;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (slices < 1 || tiles * slices > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch ||
      (slices > 1 && p.batch != 1))
    return hipErrorInvalidConfiguration;
  if (slices > 1) {
    // every slice non-empty and whole K-tiles except the last
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
      reinterpret_cast<const void*>(
          &mfma_gemm_kernel<BM, BN, BK, WM, WN, VA, VB, kMinWaves, SCHED>),
      dim3((unsigned)(tiles * slices), 1, (unsigned)p.batch), dim3(C_::kThreads), args, 0, s);
  if (err != hipSuccess || slices == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: mfma_<BM>x<BN>x<BK>_w<WM>x<WN><schedule>_<load widths>.  The default
// build holds the tiles the tuning table can pick, with 128-bit loads of A and
// B (which take any 4-byte aligned operands); a build with GEMM_F32_SWEEP
// also holds the variants that tuning sweeps compare them with.
#define GEMMF32_MFMA_VEC(BM, BN, BK, WM, WN, MW, SC, TAG)                                     \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN TAG "_vec", BM, BN, BK, WM, WN, true, true,    \
   false, &launch<BM, BN, BK, WM, WN, true, true, MW, SC>}
#define GEMMF32_MFMA_S(BM, BN, BK, WM, WN, MW, SC, TAG)                                      \
  GEMMF32_MFMA_VEC(BM, BN, BK, WM, WN, MW, SC, TAG),                                          \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN TAG "_veca", BM, BN, BK, WM, WN, true, false,  \
   false, &launch<BM, BN, BK, WM, WN, true, false, MW, SC>},                                   \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN TAG "_vecb", BM, BN, BK, WM, WN, false, true,  \
   false, &launch<BM, BN, BK, WM, WN, false, true, MW, SC>},                                   \
  {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN TAG "_scalar", BM, BN, BK, WM, WN, false,     \
   false, false, &launch<BM, BN, BK, WM, WN, false, false, MW, SC>}
#define GEMMF32_MFMA(BM, BN, BK, WM, WN, MW) GEMMF32_MFMA_S(BM, BN, BK, WM, WN, MW, 0, "")

const MfmaVariant kVariants[] = {
    // operands the direct-to-LDS loads cannot take (any pitch, 4-byte aligned)
    GEMMF32_MFMA_VEC(128, 128, 32, 64, 64, 2, 5, "_p5"),
    GEMMF32_MFMA_VEC(128, 192, 32, 32, 96, 2, 5, "_p5"),
    GEMMF32_MFMA_VEC(192, 128, 32, 96, 32, 2, 5, "_p5"),
    GEMMF32_MFMA_VEC(64, 64, 32, 32, 32, 4, 5, "_p5"),
#if GEMM_F32_SWEEP
    // the other load widths of the tiles above
    {"mfma_128x128x32_w64x64_p5_veca", 128, 128, 32, 64, 64, true, false, false,
     &launch<128, 128, 32, 64, 64, true, false, 2, 5>},
    {"mfma_128x128x32_w64x64_p5_vecb", 128, 128, 32, 64, 64, false, true, false,
     &launch<128, 128, 32, 64, 64, false, true, 2, 5>},
    {"mfma_128x128x32_w64x64_p5_scalar", 128, 128, 32, 64, 64, false, false, false,
     &launch<128, 128, 32, 64, 64, false, false, 2, 5>},
    {"mfma_64x64x32_w32x32_p5_veca", 64, 64, 32, 32, 32, true, false, false,
     &launch<64, 64, 32, 32, 32, true, false, 4, 5>},
    {"mfma_64x64x32_w32x32_p5_vecb", 64, 64, 32, 32, 32, false, true, false,
     &launch<64, 64, 32, 32, 32, false, true, 4, 5>},
    {"mfma_64x64x32_w32x32_p5_scalar", 64, 64, 32, 32, 32, false, false, false,
     &launch<64, 64, 32, 32, 32, false, false, 4, 5>},
    {"mfma_128x192x32_w32x96_p5_veca", 128, 192, 32, 32, 96, true, false, false,
     &launch<128, 192, 32, 32, 96, true, false, 2, 5>},
    {"mfma_128x192x32_w32x96_p5_vecb", 128, 192, 32, 32, 96, false, true, false,
     &launch<128, 192, 32, 32, 96, false, true, 2, 5>},
    {"mfma_128x192x32_w32x96_p5_scalar", 128, 192, 32, 32, 96, false, false, false,
     &launch<128, 192, 32, 32, 96, false, false, 2, 5>},
    {"mfma_192x128x32_w96x32_p5_veca", 192, 128, 32, 96, 32, true, false, false,
     &launch<192, 128, 32, 96, 32, true, false, 2, 5>},
    {"mfma_192x128x32_w96x32_p5_vecb", 192, 128, 32, 96, 32, false, true, false,
     &launch<192, 128, 32, 96, 32, false, true, 2, 5>},
    {"mfma_192x128x32_w96x32_p5_scalar", 192, 128, 32, 96, 32, false, false, false,
     &launch<192, 128, 32, 96, 32, false, false, 2, 5>},
    // tiles and schedules measured against them
    GEMMF32_MFMA(256, 256, 16, 128, 128, 1),
    GEMMF32_MFMA(256, 256, 32, 128, 128, 1),
    GEMMF32_MFMA(256, 128, 16, 128, 64, 2),
    GEMMF32_MFMA(128, 256, 16, 64, 128, 2),
    GEMMF32_MFMA(128, 128, 16, 64, 64, 4),
    GEMMF32_MFMA(128, 128, 32, 64, 64, 2),
    GEMMF32_MFMA(128, 64, 16, 64, 32, 4),
    GEMMF32_MFMA(64, 64, 16, 32, 32, 4),
    GEMMF32_MFMA_S(128, 128, 16, 64, 64, 4, 1, "_s1"),
    GEMMF32_MFMA_S(128, 128, 16, 64, 64, 4, 2, "_s2"),
    GEMMF32_MFMA_S(128, 128, 32, 64, 64, 2, 1, "_s1"),
    GEMMF32_MFMA_S(256, 256, 32, 128, 128, 1, 1, "_s1"),
    GEMMF32_MFMA_S(256, 128, 16, 128, 64, 2, 1, "_s1"),
    GEMMF32_MFMA_S(128, 256, 16, 64, 128, 2, 1, "_s1"),
    GEMMF32_MFMA_S(128, 128, 16, 64, 64, 3, 3, "_p3"),
    GEMMF32_MFMA_S(128, 128, 16, 64, 64, 3, 4, "_p4"),
    GEMMF32_MFMA_S(128, 128, 32, 64, 64, 2, 3, "_p3"),
    GEMMF32_MFMA_S(128, 128, 32, 64, 64, 2, 4, "_p4"),
    GEMMF32_MFMA_S(256, 128, 16, 128, 64, 2, 3, "_p3"),
    GEMMF32_MFMA_S(256, 128, 32, 128, 64, 1, 3, "_p3"),
    GEMMF32_MFMA_S(128, 64, 16, 64, 32, 4, 3, "_p3"),
    GEMMF32_MFMA_S(128, 64, 32, 64, 32, 4, 3, "_p3"),
    GEMMF32_MFMA_S(64, 64, 16, 32, 32, 4, 3, "_p3"),
    GEMMF32_MFMA_S(64, 64, 32, 32, 32, 4, 3, "_p3"),
    GEMMF32_MFMA_S(128, 128, 64, 64, 64, 1, 3, "_p3"),
    GEMMF32_MFMA_S(128, 64, 64, 64, 32, 1, 3, "_p3"),
    GEMMF32_MFMA_S(64, 64, 64, 32, 32, 2, 3, "_p3"),
    GEMMF32_MFMA_S(128, 128, 64, 64, 64, 1, 5, "_p5"),
    GEMMF32_MFMA_S(128, 128, 16, 64, 64, 3, 5, "_p5"),
    GEMMF32_MFMA_S(256, 128, 16, 128, 64, 2, 5, "_p5"),
    GEMMF32_MFMA_S(256, 128, 32, 128, 64, 1, 5, "_p5"),
    GEMMF32_MFMA_S(128, 64, 32, 64, 32, 4, 5, "_p5"),
    GEMMF32_MFMA_S(128, 64, 64, 64, 32, 1, 5, "_p5"),
    GEMMF32_MFMA_S(64, 64, 64, 32, 32, 2, 5, "_p5"),
    GEMMF32_MFMA_S(128, 192, 16, 64, 96, 1, 5, "_p5"),
    GEMMF32_MFMA_S(128, 192, 32, 64, 96, 1, 5, "_p5"),
    GEMMF32_MFMA_S(256, 192, 16, 128, 96, 1, 5, "_p5"),
    GEMMF32_MFMA_S(128, 192, 32, 32, 96, 2, 3, "_p3"),
#endif
};

}  // namespace

int mfma_variant_count() {
  return (int)(sizeof(kVariants) / sizeof(kVariants[0])) + mfma_dma_variant_count() +
         mfma_small_variant_count() + mfma_dma_ks_variant_count() + mfma_d4_variant_count();
}
const MfmaVariant& mfma_variant(int i) {
  const int n = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
  if (i < n) return kVariants[i];
  i -= n;
  if (i < mfma_dma_variant_count()) return mfma_dma_variant(i);
  i -= mfma_dma_variant_count();
  if (i < mfma_small_variant_count()) return mfma_small_variant(i);
  i -= mfma_small_variant_count();
  if (i < mfma_dma_ks_variant_count()) return mfma_dma_ks_variant(i);
  return mfma_d4_variant(i - mfma_dma_ks_variant_count());
}

}  // namespace gemmf32
