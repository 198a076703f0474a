// Skinny-M fp32 GEMM (M <= 16) reading B in whole row runs.
//
// For a few rows of A the product is a stream over B: each element of B is
// used at most 16 times, so the time is reading B once from HBM.  This kernel
// is for B stored K x N with N and the pitch multiples of 4 and B 16-byte
// aligned.  Every load of a wave then reads one contiguous run of one row of
// B: 64 lanes x VW consecutive columns (VW = 4: 1 KiB, VW = 2: 512 bytes), and
// the waves of a workgroup read neighbouring runs or neighbouring rows.  On
// MI355X a 512-byte run per wave load, eight rows in flight per wave and four
// K slices of 128-column strips (256 workgroups for N = 8192) read B at the
// rate of a plain contiguous stream; more bytes in flight per workgroup is
// slower, not faster.
//
// The contraction runs on v_mfma_f32_4x4x1_16b_f32, 16 independent 4x4x1
// outer products per instruction.  Read as C^T = B^T A^T:
//   MFMA A operand, lane l: B[k][n0 + VW l + c]           (block l/4, row l%4)
//   MFMA B operand, lane l: A[4 h + l % 4][k]             (block l/4, col l%4)
//   accumulator register r of lane l, for column phase c and row quad h:
//     C[4 h + l % 4][n0 + 4 VW (l / 4) + VW r + c]
// so one load of B feeds VW MFMAs per quad of rows of A, and the registers of
// the VW column phases are 4 VW consecutive columns of C.
// (Lane maps checked on MI355X with an index probe.)
//
// Work split: a workgroup owns CG x 64 VW columns and one K slice; its waves
// are CG column groups x RG row groups, and row group g takes the quads of
// four rows g, g + RG, ... of the slice.  The slice of A (zero-padded to 4 MQ
// rows and to whole quads) is staged in LDS once; the first loads of B are
// issued before it so the stream starts at once.  The row groups are added
// in LDS in row-group order; the slice result goes to C (one slice) or to the
// slice's partial sums, which the combine kernel adds in slice order -- the
// "combine groups" second pass of "GPU compute shaders" (How it works, step
// 6), with a fixed order so reruns are bitwise identical (its Pitfalls).
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTargetWorkgroups = 256;
constexpr int kMaxLdsBytes = 64 * 1024;

// VW columns of one row of B from p (16-byte aligned for VW = 4, 8-byte for 2)
template <int VW>
__device__ __forceinline__ void load_run(const float* p, float (&o)[VW]) {
  if constexpr (VW == 4) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else if constexpr (VW == 2) {
    const floatx2 v = __builtin_nontemporal_load(reinterpret_cast<const floatx2*>(p));
    o[0] = v.x; o[1] = v.y;
  } else {
    static_assert(VW == 1, "1, 2 or 4 columns per lane");
    o[0] = __builtin_nontemporal_load(p);
  }
}

// CG column groups x RG row groups of waves, MQ quads of rows of A, VW
// columns per lane, ST elements of A staged per thread.
template <int CG, int RG, int MQ, int VW, int ST>
struct RowsCfg {
  static constexpr int kColsPerWave = 64 * VW;
  static constexpr int kWaves = CG * RG;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRows = 4 * MQ;                 // rows of A held (M <= kRows)
  static constexpr int kAccPerLane = MQ * VW * 4;      // [h][c] x 4 registers
  // row-group partials parked in LDS at the end (row groups 1 .. RG-1)
  static constexpr int kRedBytes = (RG - 1) * CG * kAccPerLane * 64 * 4;
  static constexpr int kQuadBytes = kRows * 4 * 4;     // A slice bytes per quad of k
  // A elements staged per thread; a slice holds at most kMaxQuads quads
  static constexpr int kStage = ST;
  static constexpr int kStageBytes = kStage * kThreads * 4;
  static constexpr int kMaxQuads = kStageBytes / kQuadBytes;
  static_assert(kRedBytes <= kMaxLdsBytes && kStageBytes <= kMaxLdsBytes,
                "staging and the row-group reduction must fit the LDS budget");
};

template <int CG, int RG, int U, int MQ, int VW, int ST, bool TA>
__global__ void __launch_bounds__(CG * RG * 64)
    skinny_rows_kernel(Problem p, int kslice, int slices, float* __restrict__ part, Epilogue ep) {
  using Cfg = RowsCfg<CG, RG, MQ, VW, ST>;
  constexpr int MR = Cfg::kRows;
  extern __shared__ __attribute__((aligned(16))) float lds[];

  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int cg = wave % CG, rg = wave / CG;
  const int n_w = (blockIdx.x * CG + cg) * Cfg::kColsPerWave;
  const int slice = blockIdx.y;
  const int kb = slice * kslice;
  const int ke = min(K, kb + kslice);
  const int nq = (ke - kb + 3) >> 2;                           // quads in the slice, >= 1
  const int my_nq = nq > rg ? (nq - rg + RG - 1) / RG : 0;     // quads of this wave

  // this lane's VW columns; past N the address is clamped (N % 4 == 0) and
  // the results of those columns are never stored
  const int ncol = n_w + VW * lane;
  const float* bcol = p.B + (ncol < N ? ncol : N - VW);
  const int64_t ldb = p.ldb;

  struct Quad {
    float b[4][VW];
  };
  // j-th quad of this wave (past the last: the last again, multiplied as zeros)
  auto load = [&](Quad& x, int j) {
    const int jj = j < my_nq ? j : (my_nq > 0 ? my_nq - 1 : 0);
    const int k = kb + 4 * (rg + RG * jj);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = k + s < ke ? k + s : ke - 1;
      load_run<VW>(bcol + kk * ldb, x.b[s]);
    }
  };

  // ---- stage this slice of A: lds[(q * MR + m) * 4 + s] = A(m, kb + 4 q + s),
  // zero for rows m >= M and for k >= ke (the plan keeps the slice within
  // kStage elements per thread).  These loads are issued before the first
  // loads of B, so waiting for them does not wait for B.
  const int64_t lda = p.lda;
  float av[Cfg::kStage];
  bool aok[Cfg::kStage];
#pragma unroll
  for (int i = 0; i < Cfg::kStage; ++i) {
    const int e = tid + i * Cfg::kThreads;
    const int s = e & 3, m = (e >> 2) % MR, q = (e >> 2) / MR;
    const int k = kb + 4 * q + s;
    const int mc = m < M ? m : M - 1, kc = k < ke ? k : ke - 1;   // in-bounds address
    av[i] = TA ? p.A[(int64_t)kc * lda + mc] : p.A[(int64_t)mc * lda + kc];
    aok[i] = m < M && k < ke;
  }
  __builtin_amdgcn_sched_barrier(0);

  Quad x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) load(x[u], u);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < Cfg::kStage; ++i) {
    // the loads above are unconditional: the value is consumed here, after
    // the loads of B, so it cannot be sunk into a branch of its own
    asm volatile("" : "+v"(av[i]));
    lds[tid + i * Cfg::kThreads] = aok[i] ? av[i] : 0.f;
  }
  __syncthreads();

  floatx4 acc[MQ][VW];
#pragma unroll
  for (int h = 0; h < MQ; ++h)
#pragma unroll
    for (int c = 0; c < VW; ++c) acc[h][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int mlane = lane & 3;
  auto compute = [&](const Quad& xq, int j) {
    const bool jv = j < my_nq;                 // the same for the whole wave
    const int q = rg + RG * (jv ? j : 0);
    const int k0 = kb + 4 * q;
    floatx4 a[MQ];
#pragma unroll
    for (int h = 0; h < MQ; ++h)
      a[h] = *reinterpret_cast<const floatx4*>(&lds[(q * MR + 4 * h + mlane) * 4]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // rows past the slice (a clamped re-read) contribute exact zeros
      const bool ok = jv && (k0 + s < ke);
#pragma unroll
      for (int c = 0; c < VW; ++c) {
        const float bv = ok ? xq.b[s][c] : 0.f;
#pragma unroll
        for (int h = 0; h < MQ; ++h)
          acc[h][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(bv, ok ? a[h][s] : 0.f, acc[h][c],
                                                          0, 0, 0);
      }
    }
  };

  // Each quad is multiplied and its registers refilled with the quad U ahead,
  // so U quads stay in flight.  The last two rounds refill only quads that
  // exist: B is read once, with no loads past the slice.
  int j0 = 0;
  for (; j0 + 2 * U <= my_nq; j0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      compute(x[u], j0 + u);
      load(x[u], j0 + u + U);
      // keep the rotation in program order: the other U - 1 quads stay in
      // flight while this one is multiplied
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    compute(x[u], j0 + u);
    if (j0 + u + U < my_nq) load(x[u], j0 + u + U);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (j0 + U + u < my_nq) compute(x[u], j0 + U + u);

  // ---- add the row groups in row-group order (LDS reused) -------------------
  if (RG > 1) {
    __syncthreads();   // every wave is done with the staged A
    if (rg > 0) {
      float* red = lds + ((rg - 1) * CG + cg) * Cfg::kAccPerLane * 64;
#pragma unroll
      for (int h = 0; h < MQ; ++h)
#pragma unroll
        for (int c = 0; c < VW; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((h * VW + c) * 4 + r) * 64 + lane] = acc[h][c][r];
    }
    __syncthreads();
    if (rg > 0) return;
#pragma unroll
    for (int g = 1; g < RG; ++g) {
      const float* red = lds + ((g - 1) * CG + cg) * Cfg::kAccPerLane * 64;
#pragma unroll
      for (int h = 0; h < MQ; ++h)
#pragma unroll
        for (int c = 0; c < VW; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[h][c][r] += red[((h * VW + c) * 4 + r) * 64 + lane];
    }
  }

  // ---- write: lane l holds C[4 h + l % 4][n_w + 4 VW (l / 4) + VW r + c] -----
  const int nb = n_w + 4 * VW * (lane >> 2);
#pragma unroll
  for (int h = 0; h < MQ; ++h) {
    const int m = 4 * h + mlane;
    if (m >= M) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = nb + VW * r;
      // N % 4 == 0 and n % VW == 0: the VW columns are all in or all out
      if (n >= N) continue;
      if (slices == 1) {
        // C = act(alpha * sum + beta * C + bias) (C not read when beta == 0)
        float* d = p.C + (int64_t)m * p.ldc + n;
#pragma unroll
        for (int c = 0; c < VW; ++c) d[c] = epilogue_apply(ep, acc[h][c][r], d + c, n + c);
      } else {
        // aligned to 4 VW bytes: N % 4 == 0 and n % VW == 0
        float* d = part + ((size_t)slice * M + m) * N + n;
        if constexpr (VW == 4) {
          *reinterpret_cast<floatx4*>(d) =
              floatx4{acc[h][0][r], acc[h][1][r], acc[h][2][r], acc[h][3][r]};
        } else if constexpr (VW == 2) {
          *reinterpret_cast<floatx2*>(d) = floatx2{acc[h][0][r], acc[h][1][r]};
        } else {
          *d = acc[h][0][r];
        }
      }
    }
  }
}

// Slices: enough workgroups for every CU (or `target` slices), each slice at
// least 4 quads per row group, and its staged A within the LDS budget.
template <int CG, int RG, int MQ, int VW, int ST>
SkinnyPlan plan_rows(const Problem& p, int target) {
  using Cfg = RowsCfg<CG, RG, MQ, VW, ST>;
  SkinnyPlan pl{};
  constexpr int kCols = CG * Cfg::kColsPerWave;
  pl.strips = (p.N + kCols - 1) / kCols;
  const int64_t quads = (p.K + 3) / 4;
  int64_t slices = target > 0 ? target
                              : (kTargetWorkgroups + pl.strips - 1) / pl.strips;
  const int64_t cap = quads / (4 * RG);
  if (slices > cap) slices = cap;
  if (slices < 1) slices = 1;
  int64_t per = (quads + slices - 1) / slices;
  if (per > Cfg::kMaxQuads) per = Cfg::kMaxQuads;
  const int64_t splits = (quads + per - 1) / per;   // no empty slice
  pl.splits = splits > 65536 ? 65536 : (int)splits;   // launch rejects > 65535
  pl.kslice = (int)(per * 4);
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.lds_bytes = Cfg::kStageBytes > Cfg::kRedBytes ? Cfg::kStageBytes : Cfg::kRedBytes;
  return pl;
}

template <int CG, int RG, int U, int MQ, int VW, int ST, bool TA>
hipError_t launch_rows(const Problem& p, const SkinnyPlan& pl, float* partials,
                       const Epilogue& e, hipStream_t s) {
  using Cfg = RowsCfg<CG, RG, MQ, VW, ST>;
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.M > Cfg::kRows || p.batch != 1 ||
      p.N % 4 != 0 || p.ldb % 4 != 0 || (reinterpret_cast<uintptr_t>(p.B) & 15) != 0 ||
      pl.lds_bytes > (size_t)kMaxLdsBytes)
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !partials) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, slices = pl.splits;
  float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &kslice, &slices, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_rows_kernel<CG, RG, U, MQ, VW, ST, TA>),
      dim3(pl.strips, pl.splits), dim3(Cfg::kThreads), args, pl.lds_bytes, s);
  if (err != hipSuccess || pl.splits == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: skinnyr_c<column groups of 64 VW>_r<row groups>_u<quads in flight>_m<rows
// of A>[_v<VW>]_s<K slices, 0 = from the shape>_<nn|tn>; without _v, VW = 4.
#define GEMMF32_SKINNY_ROWS_NN(CG, RG, U, MQ, VW, ST, S, VS)                                 \
  {"skinnyr_c" #CG "_r" #RG "_u" #U "_m" #MQ "x4" VS "_s" #S "_nn", 4 * MQ, CG * RG, U,       \
   false, true, S, false, false, &plan_rows<CG, RG, MQ, VW, ST>,                              \
   &launch_rows<CG, RG, U, MQ, VW, ST, false>, true}
#define GEMMF32_SKINNY_ROWS_TN(CG, RG, U, MQ, VW, ST, S, VS)                                 \
  {"skinnyr_c" #CG "_r" #RG "_u" #U "_m" #MQ "x4" VS "_s" #S "_tn", 4 * MQ, CG * RG, U,       \
   false, true, S, true, false, &plan_rows<CG, RG, MQ, VW, ST>,                               \
   &launch_rows<CG, RG, U, MQ, VW, ST, true>, true}
#define GEMMF32_SKINNY_ROWS_V(CG, RG, U, MQ, VW, ST, S, VS) \
  GEMMF32_SKINNY_ROWS_NN(CG, RG, U, MQ, VW, ST, S, VS), GEMMF32_SKINNY_ROWS_TN(CG, RG, U, MQ, VW, ST, S, VS)
#define GEMMF32_SKINNY_ROWS(CG, RG, U, MQ, S) GEMMF32_SKINNY_ROWS_V(CG, RG, U, MQ, 4, 8, S, "")

// The default build holds the kernel the tuning table picks (A as stored); a
// build with GEMM_F32_SWEEP also holds the ones tuning sweeps compared it with.
const SkinnyVariant kRowsVariants[] = {
    GEMMF32_SKINNY_ROWS_NN(2, 4, 4, 2, 4, 8, 0, ""),
#if GEMM_F32_SWEEP
    GEMMF32_SKINNY_ROWS_TN(2, 4, 4, 2, 4, 8, 0, ""),
    GEMMF32_SKINNY_ROWS(2, 4, 2, 2, 0),
    GEMMF32_SKINNY_ROWS(4, 2, 2, 2, 0),
    GEMMF32_SKINNY_ROWS(4, 1, 4, 2, 0),
    GEMMF32_SKINNY_ROWS(1, 8, 2, 2, 8),
    GEMMF32_SKINNY_ROWS(4, 2, 2, 4, 0),
    GEMMF32_SKINNY_ROWS(4, 2, 4, 1, 0),
    // 512-byte runs (two columns per lane), the slice of A staged whole
    GEMMF32_SKINNY_ROWS_V(1, 8, 2, 2, 2, 32, 0, "_v2"),
    GEMMF32_SKINNY_ROWS_V(1, 8, 1, 2, 2, 32, 0, "_v2"),
    GEMMF32_SKINNY_ROWS_V(1, 8, 3, 2, 2, 32, 0, "_v2"),
    GEMMF32_SKINNY_ROWS_V(1, 4, 4, 2, 2, 32, 0, "_v2"),
    GEMMF32_SKINNY_ROWS_V(1, 4, 2, 2, 2, 32, 0, "_v2"),
    // 256-byte runs
    GEMMF32_SKINNY_ROWS_V(1, 8, 2, 2, 1, 32, 0, "_v1"),
    GEMMF32_SKINNY_ROWS_V(1, 8, 4, 2, 1, 32, 0, "_v1"),
#endif
};

}  // namespace

int skinny_rows_variant_count() {
  return (int)(sizeof(kRowsVariants) / sizeof(kRowsVariants[0]));
}
const SkinnyVariant& skinny_rows_variant(int i) { return kRowsVariants[i]; }

}  // namespace gemmf32
