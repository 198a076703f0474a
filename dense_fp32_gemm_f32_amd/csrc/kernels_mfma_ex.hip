// Macro-tiled fp32 MFMA GEMM for the extended operation
//   C = alpha * op(A) op(B) + beta * C,  op(X) = X or X^T (row-major storage).
//
// The pages multiply row-major A and B; "Optimizing a WebGPU Matmul Kernel
// using Subgroups" (section 7) also feeds a pre-transposed B.  Here either
// operand may be stored either way.  The MFMA operands of
// v_mfma_f32_32x32x2_f32 are symmetric -- lane l of the A operand holds
// A[l % 32][k-slot l / 32] and lane l of the B operand holds B[k-slot l / 32]
// [l % 32] -- so one operand description serves A (rows = m) and B (rows =
// n), in one of two storage layouts:
//   KC  ("k contiguous"): element (r, k) at X[r * ld + k]   (A as is, B^T)
//   RC  ("r contiguous"): element (r, k) at X[k * ld + r]   (A^T, B as is)
// Tiles and schedule follow the register-staged kernel (kernels_mfma.hip):
// 128-bit global loads (dword alignment suffices), LDS double buffer with one
// barrier per K-tile, fragments read one k group ahead, global loads two
// K-tiles ahead, and a branch-free loop for the K-tiles inside K in which each
// memory instruction follows its own MFMA.  In LDS a KC operand is stored
// [r][k] with its 16-byte chunks swizzled by row (128-bit fragment reads), an
// RC operand [k][r] with r XORed by 32 on bit 2 of k (32-bit fragment reads).
#include <type_traits>

#include "gemm_f32_internal.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

using namespace mfma;

// One operand's share of a K-tile: R rows (BM for A, BN for B) by BK.
template <int R, int BK, int kThreads, bool KC>
struct Operand {
  static constexpr int kChunks = R * BK / 4;
  static constexpr int kPer = kChunks / kThreads;   // 16-byte chunks per thread
  static constexpr int kLds = R * BK;
  static constexpr int kRowChunks = KC ? BK / 4 : R / 4;
  static_assert(kChunks % kThreads == 0, "chunks divide evenly over the threads");
  static_assert(KC || R % 64 == 0, "the [k][r] swizzle needs 64-wide rows");
  static_assert(!KC || BK / 4 <= 16, "the [r][k] swizzle covers at most 16 chunks");

  const float* ptr[kPer];   // first element of each chunk at K-tile 0 (clamped)
  int r_of[kPer];           // tile row of the chunk's first element
  int k_of[kPer];           // K-tile row of the chunk's first element
  float4 reg[kPer];         // staging registers

  // Chunk e of the tile: (r, k) of its first element.
  __device__ __forceinline__ static void chunk_rk(int e, int& r, int& k) {
    if (KC) {
      r = e / kRowChunks;
      k = 4 * (e % kRowChunks);
    } else {
      k = e / kRowChunks;
      r = 4 * (e % kRowChunks);
    }
  }
  __device__ __forceinline__ static int lds_off(int r, int k) {
    return KC ? r * BK + 4 * ((k / 4) ^ swz_a<BK / 4>(r)) : k * R + (r ^ swz_b(k));
  }

  // base: the operand; ld: its pitch; r0: first tile row; rtot: M or N.
  __device__ __forceinline__ void init(const float* base, int64_t ld, int r0, int rtot,
                                       int tid) {
#pragma unroll
    for (int v = 0; v < kPer; ++v) {
      int r, k;
      chunk_rk(tid + v * kThreads, r, k);
      r_of[v] = r;
      k_of[v] = k;
      const int gr = r0 + r;
      if (KC) {
        ptr[v] = base + (int64_t)(gr < rtot ? gr : r0) * ld + k;
      } else {
        ptr[v] = base + (int64_t)k * ld + (gr < rtot ? gr : r0);
      }
    }
  }
  __device__ __forceinline__ static int64_t kstep(int64_t ld, int k0) {
    return KC ? (int64_t)k0 : (int64_t)k0 * ld;
  }

  // K-tile at k0 lies inside K.  Rows past rtot are read at clamped addresses
  // and reach only rows or columns of C that are not stored.  EDGE (RC only):
  // a chunk of this tile straddles rtot (rtot % 4 != 0), so every chunk is
  // read element by element with its row clamped to rtot - 1.
  template <bool EDGE>
  __device__ __forceinline__ void load_fast(int v, int64_t ld, int k0, int r0, int rtot) {
    const float* src = ptr[v] + kstep(ld, k0);
    if (!KC && EDGE) {
      const float* row = src - ((r0 + r_of[v] < rtot) ? r_of[v] : 0);   // element r0 of this k row
      const int gr = r0 + r_of[v], last = rtot - 1;
      reg[v] = make_float4(row[min(gr, last) - r0], row[min(gr + 1, last) - r0],
                           row[min(gr + 2, last) - r0], row[min(gr + 3, last) - r0]);
    } else {
      reg[v] = load4(src);
    }
  }
  // Any K-tile: elements outside rtot x K become 0.0.
  __device__ __forceinline__ void load_masked(int v, int64_t ld, int k0, int K, int r0,
                                              int rtot) {
    const int gr = r0 + r_of[v], gk = k0 + k_of[v];
    if (KC) {
      const float* src = ptr[v] + k0;
      const bool ok = gr < rtot;
      if (ok && gk + 3 < K) {
        reg[v] = load4(src);
      } else {
        reg[v].x = (ok && gk + 0 < K) ? src[0] : 0.f;
        reg[v].y = (ok && gk + 1 < K) ? src[1] : 0.f;
        reg[v].z = (ok && gk + 2 < K) ? src[2] : 0.f;
        reg[v].w = (ok && gk + 3 < K) ? src[3] : 0.f;
      }
    } else {
      const bool kok = gk < K;
      const float* row = ptr[v] + (int64_t)k0 * ld - ((gr < rtot) ? r_of[v] : 0);
      if (kok && gr + 3 < rtot) {
        reg[v] = load4(row + r_of[v]);
      } else {
        reg[v].x = (kok && gr + 0 < rtot) ? row[r_of[v] + 0] : 0.f;
        reg[v].y = (kok && gr + 1 < rtot) ? row[r_of[v] + 1] : 0.f;
        reg[v].z = (kok && gr + 2 < rtot) ? row[r_of[v] + 2] : 0.f;
        reg[v].w = (kok && gr + 3 < rtot) ? row[r_of[v] + 3] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(float* lds, int v) const {
    *reinterpret_cast<float4*>(&lds[lds_off(r_of[v], k_of[v])]) = reg[v];
  }
};

// Fragments of one 8-wide k group for FR 32-row blocks of one operand.
template <int FR, bool KC>
struct Frag {
  float v[4][FR];   // [MFMA step s][block]
};

template <int BM, int BN, int BK, int WM, int WN, bool A_KC, bool B_KC, int kMinWaves>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(kMinWaves)))
    mfma_ex_kernel(Problem p, Epilogue e, int tiles_m, int tiles_n) {
  constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  constexpr int kThreads = kWavesM * kWavesN * 64;
  constexpr int kFragM = WM / 32, kFragN = WN / 32;
  using OpA = Operand<BM, BK, kThreads, A_KC>;
  using OpB = Operand<BN, BK, kThreads, B_KC>;
  static_assert(BK % 16 == 0, "BK in {16, 32, 64}");
  __shared__ __attribute__((aligned(16))) float lds_a[2][OpA::kLds];
  __shared__ __attribute__((aligned(16))) float lds_b[2][OpB::kLds];

  const int tid = threadIdx.x;
  select_batch(p);
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  OpA opa;
  OpB opb;
  opa.init(p.A, p.lda, m0, M, tid);
  opb.init(p.B, p.ldb, n0, N, tid);
  constexpr int kLoads = OpA::kPer + OpB::kPer;

  auto load_masked = [&](int k0) {
#pragma unroll
    for (int v = 0; v < OpA::kPer; ++v) opa.load_masked(v, p.lda, k0, K, m0, M);
#pragma unroll
    for (int v = 0; v < OpB::kPer; ++v) opb.load_masked(v, p.ldb, k0, K, n0, N);
  };
  auto store_all = [&](int buf) {
#pragma unroll
    for (int v = 0; v < OpA::kPer; ++v) opa.store(lds_a[buf], v);
#pragma unroll
    for (int v = 0; v < OpB::kPer; ++v) opb.store(lds_b[buf], v);
  };
  auto store_one = [&](int buf, int idx) {
    if (idx < OpA::kPer) {
      opa.store(lds_a[buf], idx);
    } else {
      opb.store(lds_b[buf], idx - OpA::kPer);
    }
  };
  // global load idx of a K-tile inside K (edge: straddling RC chunks)
  auto load_one_fast = [&](int k0, int idx, auto ea_tag, auto eb_tag) {
    if (idx < OpA::kPer) {
      opa.template load_fast<decltype(ea_tag)::value>(idx, p.lda, k0, m0, M);
    } else {
      opb.template load_fast<decltype(eb_tag)::value>(idx - OpA::kPer, p.ldb, k0, n0, N);
    }
  };

  // ---- fragments --------------------------------------------------------
  const int wave = tid >> 6, lane = tid & 63;
  const int wmi = wave % kWavesM, wni = wave / kWavesM;
  const int lr = lane & 31, lk = lane >> 5;
  // fragment of block i (rows base + 32 i + lr), group q, for each step s
  auto read_op = [&](auto& f, const float* lds, int rbase, int R, bool kc, int q, int i) {
    const int r = rbase + 32 * i + lr;
    if (kc) {
      const int off = r * BK + 4 * ((2 * q + lk) ^ swz_a<BK / 4>(r));
      const float4 t = *reinterpret_cast<const float4*>(&lds[off]);
      f.v[0][i] = t.x;
      f.v[1][i] = t.y;
      f.v[2][i] = t.z;
      f.v[3][i] = t.w;
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) f.v[s][i] = lds[(8 * q + 4 * lk + s) * R + (r ^ (lk << 5))];
    }
  };
  using FA = Frag<kFragM, A_KC>;
  using FB = Frag<kFragN, B_KC>;
  // op index -> one block of A or of B
  constexpr int kReads = kFragM + kFragN;
  auto read_one = [&](FA& fa, FB& fb, int buf, int q, int idx) {
    if (idx < kFragM) {
      read_op(fa, lds_a[buf], wmi * WM, BM, A_KC, q, idx);
    } else {
      read_op(fb, lds_b[buf], wni * WN, BN, B_KC, q, idx - kFragM);
    }
  };

  floatx16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr int kMfma = 4 * kFragM * kFragN;
  auto mfma_one = [&](const FA& fa, const FB& fb, int idx) {
    const int s = idx / (kFragM * kFragN);
    const int i = (idx / kFragN) % kFragM, j = idx % kFragN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.v[s][i], fb.v[s][j], acc[i][j], 0, 0, 0);
  };

  // ---- K loop (as SCHED 5 of the register-staged kernel) -----------------
  constexpr int kGroups = BK / 8;
  constexpr int kStoreQ = kGroups - 2;
  constexpr int kHalf = kMfma / 2;
  const int ktiles = (K + BK - 1) / BK;
  FA fa0, fa1;
  FB fb0, fb1;
  load_masked(0);
  store_all(0);
  __syncthreads();
#pragma unroll
  for (int idx = 0; idx < kReads; ++idx) read_one(fa0, fb0, 0, 0, idx);
  if (ktiles > 1) load_masked(BK);

  auto step = [&](int t, auto fast_tag, auto ea_tag, auto eb_tag) {
    constexpr bool kFast = decltype(fast_tag)::value;
    const int cur = t & 1;
    const bool more = kFast || t + 1 < ktiles;
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      FA& fac = (q & 1) ? fa1 : fa0;
      FB& fbc = (q & 1) ? fb1 : fb0;
      FA& fan = (q & 1) ? fa0 : fa1;
      FB& fbn = (q & 1) ? fb0 : fb1;
      if (q < kGroups - 1) {
        if constexpr (kFast) {
          constexpr int kWritesPer = (kLoads + kMfma - 1) / kMfma;
#pragma unroll
          for (int i = 0; i < kMfma; ++i) {
            mfma_one(fac, fbc, i);
            if (i < kReads) read_one(fan, fbn, cur, q + 1, i);
            if (q == kStoreQ) {
#pragma unroll
              for (int w = 0; w < kWritesPer; ++w)
                if (i * kWritesPer + w < kLoads) store_one(cur ^ 1, i * kWritesPer + w);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int idx = 0; idx < kReads; ++idx) read_one(fan, fbn, cur, q + 1, idx);
          if (q == kStoreQ && more) store_all(cur ^ 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < kMfma; ++i) mfma_one(fac, fbc, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kHalf; ++i) mfma_one(fac, fbc, i);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if constexpr (kFast) {
          constexpr int kLoadsPer = (kLoads + kHalf - 1) / kHalf;
          constexpr int kReadsPer = (kReads + kHalf - 1) / kHalf;
#pragma unroll
          for (int i = 0; i < kHalf; ++i) {
            mfma_one(fac, fbc, kHalf + i);
#pragma unroll
            for (int r = 0; r < kReadsPer; ++r)
              if (i * kReadsPer + r < kReads) read_one(fan, fbn, cur ^ 1, 0, i * kReadsPer + r);
#pragma unroll
            for (int l = 0; l < kLoadsPer; ++l)
              if (i * kLoadsPer + l < kLoads)
                load_one_fast((t + 2) * BK, i * kLoadsPer + l, ea_tag, eb_tag);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          if (more) {
#pragma unroll
            for (int idx = 0; idx < kReads; ++idx) read_one(fan, fbn, cur ^ 1, 0, idx);
            if (t + 2 < ktiles) load_masked((t + 2) * BK);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = kHalf; i < kMfma; ++i) mfma_one(fac, fbc, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  static_assert(kGroups % 2 == 0, "fragment ping-pong needs an even group count");

  int t = 0;
  {
    // an RC operand with a chunk straddling its edge reads element by element
    const int kfull = K / BK;
    const bool edge = (!A_KC && m0 + BM > M && M % 4 != 0) || (!B_KC && n0 + BN > N && N % 4 != 0);
    using T = std::true_type;
    using F = std::false_type;
    if (!edge) {
      for (; t + 2 < kfull; ++t) step(t, T{}, F{}, F{});
    } else {
      for (; t + 2 < kfull; ++t) step(t, T{}, T{}, T{});
    }
  }
  for (; t < ktiles; ++t) step(t, std::false_type{}, std::false_type{}, std::false_type{});

  // ---- epilogue: C = act(alpha * acc + beta * C + bias) (C not read when beta == 0)
  store_blocks<kFragM, kFragN>(acc, p.C, p.ldc, M, N, m0 + wmi * WM, n0 + wni * WN, lane, false,
                               e);
}

template <int BM, int BN, int BK, int WM, int WN, bool A_KC, bool B_KC, int kMinWaves>
hipError_t launch_ex(const Problem& p, const Epilogue& e, hipStream_t s) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles > 0x7fffffff || p.batch < 1 || p.batch > kMaxLaunchBatch)
    return hipErrorInvalidConfiguration;
  Problem pp = p;
  Epilogue ee = e;
  int tm = tiles_m, tn = tiles_n;
  void* args[] = {&pp, &ee, &tm, &tn};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&mfma_ex_kernel<BM, BN, BK, WM, WN, A_KC, B_KC, kMinWaves>),
      dim3((unsigned)tiles, 1, (unsigned)p.batch), dim3((BM / WM) * (BN / WN) * 64), args, 0,
      s);
}

// Name: mfmaex_<tile>_<layout>, layout = op(A) op(B) as n (stored as is) or t
// (stored transposed).  A is KC when not transposed; B is KC when transposed.
// The default build holds the tiles the tuning table can pick, in the three
// layouts with a transposed operand (A and B as stored run the plain
// kernels); a build with GEMM_F32_SWEEP adds the _nn twins and the other tiles.
#define GEMMF32_MFMA_EX_T(BM, BN, BK, WM, WN, MW)                                        \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_nt", BM, BN, BK, false, true,       \
   &launch_ex<BM, BN, BK, WM, WN, true, true, MW>},                                      \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_tn", BM, BN, BK, true, false,       \
   &launch_ex<BM, BN, BK, WM, WN, false, false, MW>},                                    \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_tt", BM, BN, BK, true, true,        \
   &launch_ex<BM, BN, BK, WM, WN, false, true, MW>}
#define GEMMF32_MFMA_EX_NN(BM, BN, BK, WM, WN, MW)                                       \
  {"mfmaex_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_nn", BM, BN, BK, false, false,      \
   &launch_ex<BM, BN, BK, WM, WN, true, false, MW>}

const MfmaExVariant kExVariants[] = {
    GEMMF32_MFMA_EX_T(128, 128, 16, 64, 64, 2),
    GEMMF32_MFMA_EX_T(128, 64, 32, 64, 32, 2),
    GEMMF32_MFMA_EX_T(64, 64, 32, 32, 32, 2),
#if GEMM_F32_SWEEP
    GEMMF32_MFMA_EX_NN(128, 128, 16, 64, 64, 2),
    GEMMF32_MFMA_EX_NN(128, 64, 32, 64, 32, 2),
    GEMMF32_MFMA_EX_NN(64, 64, 32, 32, 32, 2),
    GEMMF32_MFMA_EX_NN(256, 128, 16, 128, 64, 1),
    GEMMF32_MFMA_EX_T(256, 128, 16, 128, 64, 1),
#endif
};

}  // namespace

int mfma_ex_variant_count() {
  return (int)(sizeof(kExVariants) / sizeof(kExVariants[0])) + mfma_ex_dma_variant_count();
}
const MfmaExVariant& mfma_ex_variant(int i) {
  const int n = (int)(sizeof(kExVariants) / sizeof(kExVariants[0]));
  return i < n ? kExVariants[i] : mfma_ex_dma_variant(i - n);
}

}  // namespace gemmf32
