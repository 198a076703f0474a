// Skinny-M fp32 GEMM (M <= 16): a bandwidth-bound stream over B.
//
// With few rows of A every element of B is used at most 16 times, so the time
// goes into reading B once from HBM.  Two measured facts about MI355X shape
// this kernel:
//  - B is read fastest when each workgroup streams a tile 128 columns wide
//    (512-byte row runs) with non-temporal loads; 32-column strips over all of
//    K top out near 5 TB/s, 128-column tiles over a quarter of K reach 6+ TB/s;
//  - combining partial sums of several workgroups inside one kernel needs an
//    agent-scope release per workgroup (a whole-L2 writeback on this GPU),
//    and those are serialised: about 0.16 us each, 40 us for 256 workgroups.
// So the K range is split over a few slices, and the slices' partial sums are
// added in one of two ways:
//  - each workgroup writes its slice's partial sums and a second small kernel
//    adds the slices in slice order;
//  - XCH: the slices meet in a binary tree of exchange slots inside this
//    kernel.  Per output element, the two children of a tree node each swap
//    (flag, value) into the node's 64-bit slot with one device-scope atomic
//    exchange; the one that finds the slot full holds both values, adds them
//    as left + right, empties the slot and carries the sum up.  The carrier
//    of the root applies the epilogue and writes C.  The value travels inside
//    the atomic, so no fence and no waiting on another workgroup is needed,
//    and the additions are fixed by the slice count alone.
// This is the "combine groups" step of "GPU compute shaders" (How it works,
// step 6: one partial per group, then the partials reduced); fixing the group
// count and the order of the sum keeps reruns bitwise identical, as the
// Pitfalls section of that page asks.
//
// The product inside a tile is read as C^T = B^T A^T on the matrix cores:
// v_mfma_f32_16x16x4_f32 takes 16 columns of B as its M dimension, up to 16
// rows of A as its N dimension (rows >= M are zero) and 4 rows of B / columns
// of A as its K dimension.  Operand layout (wave64):
//   A operand, lane l: B[k0 + l/16][col(l % 16)]
//   B operand, lane l: A[l % 16][k0 + l/16]
//   accumulator register r of lane l: C^T[col(4*(l/16) + r)][l % 16]
// A lane holds a single A value per 4 rows, so the registers hold B loads in
// flight instead.  This is a dense contraction, so it belongs on MFMA; the
// bound is still HBM.
#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kGroupCols = 32;   // columns per wave: 16 lanes x float2

// One wave streams 16-row super-blocks first, first + step, ... < end of its
// 32 columns [n0, n0 + 32).  In super-block j (rows k0 = 16 j .. k0 + 15)
// MFMA step s (0..3) puts row k0 + 4 kr + s in k-slot kr = lane / 16 of both
// operands, so one lane needs A[m][k0 + 4 kr .. + 3] -- one 16-byte load -- and
// four B rows.  U super-blocks are in flight; a prefetch past `end` re-reads
// super-block `first` and is multiplied as exact zeros, so the loop has no
// branch and the compiler can wait for each load precisely.  Columns past N
// are read at a clamped address and replaced by 0.0 where they are used.
// `tail`: this wave also takes the last K % 16 rows, masked element by element.
// PAIR: one 8-byte load for the lane's two columns (B and its pitch 8-byte
// aligned, N even), else two 4-byte loads.  VA: one 16-byte load of A per
// super-block (any pitch), else four 4-byte loads.
template <int U, bool PAIR, bool VA, bool TA>
__device__ __forceinline__ void stream_tile(const Problem& p, int lane, int n0, int first,
                                            int end, int step, bool tail,
                                            float (&out)[2][4]) {
  const int M = p.M, N = p.N, K = p.K;
  const int kr = lane >> 4, i16 = lane & 15;
  const int col = n0 + 2 * i16;
  const bool c0_ok = col < N, c1_ok = col + 1 < N;
  const int col_x = c0_ok ? col : N - 1;
  const int col_y = c1_ok ? col + 1 : N - 1;
  const int col_p = c0_ok ? col : N - 2;   // PAIR only: N even, so col and col + 1 agree
  const bool a_row_ok = i16 < M;
  const int64_t ldb = p.ldb;
  // element (m, k) of op(A): A[m * lda + k], or A[k * lda + m] when TA (A
  // stored K x M); arow points at (this lane's row, k = 4 kr)
  const int64_t a_kstride = TA ? p.lda : 1;
  const float* arow = TA ? p.A + (a_row_ok ? i16 : M - 1) + (int64_t)(4 * kr) * p.lda
                         : p.A + (int64_t)(a_row_ok ? i16 : M - 1) * p.lda + 4 * kr;
  const float* bl[4];   // this lane's B row s of super-block 0
#pragma unroll
  for (int s = 0; s < 4; ++s) bl[s] = p.B + (int64_t)(4 * kr + s) * ldb;

  struct SB {
    floatx2 b[4];
    float4 a;
  };
  int next = first;
  auto load = [&](SB& x) {
    const int j = next < end ? next : first;
    const int k0 = 16 * j;
    const int64_t boff = (int64_t)k0 * ldb;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* r = bl[s] + boff;
      if (PAIR) {
        x.b[s] = __builtin_nontemporal_load(reinterpret_cast<const floatx2*>(r + col_p));
      } else {
        x.b[s].x = __builtin_nontemporal_load(r + col_x);
        x.b[s].y = __builtin_nontemporal_load(r + col_y);
      }
    }
    if (TA) {
      const float* a = arow + (int64_t)k0 * a_kstride;
      x.a = make_float4(a[0], a[a_kstride], a[2 * a_kstride], a[3 * a_kstride]);
    } else if (VA) {
      // 16 bytes from a 4-byte aligned address: multi-dword global loads need
      // dword alignment only, and this copy becomes one global_load_dwordx4
      __builtin_memcpy(&x.a, arow + k0, sizeof(x.a));
    } else {
      x.a = make_float4(arow[k0], arow[k0 + 1], arow[k0 + 2], arow[k0 + 3]);
    }
    next += step;
  };

  floatx4 acc[2][2];   // [even/odd super-block][even/odd column]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[h][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  // valid: the super-block exists; k_all_ok: its 16 rows are all < K
  auto mfma4 = [&](const SB& x, int h, bool valid, bool k_all_ok, int kbase) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool k_ok = valid && (k_all_ok || (kbase + 4 * kr + s < K));
      const float bx = (k_ok && c0_ok) ? x.b[s].x : 0.f;
      const float by = (k_ok && c1_ok) ? x.b[s].y : 0.f;
      const float av0 = s == 0 ? x.a.x : s == 1 ? x.a.y : s == 2 ? x.a.z : x.a.w;
      const float av = (k_ok && a_row_ok) ? av0 : 0.f;
      acc[h][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(bx, av, acc[h][0], 0, 0, 0);
      acc[h][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(by, av, acc[h][1], 0, 0, 0);
    }
  };

  if (first < end) {
    SB x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(x[u]);
    for (int j0 = first; j0 < end; j0 += U * step) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mfma4(x[u], u & 1, j0 + u * step < end, true, 0);
        load(x[u]);
        // keep the rotation in program order: the other U - 1 super-blocks
        // stay in flight while this one is multiplied
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (tail) {
    const int k0 = 16 * (K / 16);
    SB x;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = k0 + 4 * kr + s;
      const float* r = p.B + (int64_t)(k < K ? k : K - 1) * ldb;
      x.b[s].x = r[col_x];
      x.b[s].y = r[col_y];
    }
    float av[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = k0 + 4 * kr + s;
      av[s] = arow[(int64_t)((k < K ? k : K - 1) - 4 * kr) * a_kstride];
    }
    x.a = make_float4(av[0], av[1], av[2], av[3]);
    mfma4(x, 0, true, false, k0);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[c][r] = acc[0][c][r] + acc[1][c][r];
}

// Workgroup: NW waves = CG column groups x (NW / CG) row groups; it owns the
// CG * 32 columns from blockIdx.x * CG * 32 and the super-blocks
// [sb_begin, sb_end) of its K slice (blockIdx.y).  The row groups are added in
// LDS in row-group order and the result goes to C (one slice) or to the
// slice's partial sums.
template <int NW, int CG, int U, bool VA, bool VB, bool TA, bool XCH>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 16 ? 4 : 2)))
    skinny_tile_kernel(Problem p, int sb_per_slice, int slices, float* __restrict__ part,
                       unsigned long long* __restrict__ slots, Epilogue ep) {
  constexpr int NRG = NW / CG;
  static_assert(NW % CG == 0, "whole row groups");
  __shared__ __attribute__((aligned(16))) float red[NW][2][4][64];

  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int cg = wave % CG, rg = wave / CG;
  const int n_wg = blockIdx.x * (CG * kGroupCols);
  const int slice = blockIdx.y;
  const int nsb = K / 16;
  const int sb_begin = slice * sb_per_slice;
  const int sb_end = min(nsb, sb_begin + sb_per_slice);
  // the partial super-block of rows K/16*16 .. K-1 belongs to the last slice
  const bool tail = (K % 16 != 0) && slice == slices - 1 && rg == (sb_end - sb_begin) % NRG;

  float out[2][4];
  const bool pair = VB && (N % 2) == 0 && (p.ldb % 2) == 0 &&
                    (reinterpret_cast<uintptr_t>(p.B) & 7) == 0;
  if (pair) {
    stream_tile<U, true, VA, TA>(p, lane, n_wg + cg * kGroupCols, sb_begin + rg, sb_end, NRG,
                                 tail, out);
  } else {
    stream_tile<U, false, VA, TA>(p, lane, n_wg + cg * kGroupCols, sb_begin + rg, sb_end, NRG,
                                  tail, out);
  }

#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][c][r][lane] = out[c][r];
  __syncthreads();
  float* dst;
  int64_t ld;
  if (slices == 1 || XCH) {
    dst = p.C;
    ld = p.ldc;
  } else {
    dst = part + (size_t)slice * M * N;
    ld = N;
  }
  constexpr int kTileElems = CG * 2 * 4 * 64;
  // one output per thread: column group, even/odd column, register, lane
  for (int e = tid; e < kTileElems; e += NW * 64) {
    const int g = e / 512, c = (e / 256) % 2, r = (e / 64) % 4, l = e % 64;
    const int m = l & 15;
    const int n = n_wg + g * kGroupCols + 2 * (4 * (l >> 4) + r) + c;
    if (m < M && n < N) {
      float s = red[g][c][r][l];
      for (int w = 1; w < NRG; ++w) s += red[w * CG + g][c][r][l];
      float* d = dst + (int64_t)m * ld + n;
      if (slices == 1) {
        *d = epilogue_apply(ep, s, d, n);
      } else if (!XCH) {
        *d = s;
      } else {
        // Tree over the slices: at each level node j has children 2j, 2j+1;
        // a node without a right child passes its value up unchanged.  The
        // slots of a level's nodes follow one another, node j's slot for this
        // element at ((base + j) * strips + strip) * kTileElems + e, so the
        // lanes of a wave swap consecutive words.
        int node = slice, width = slices, base = 0;
        bool carry = true;
        while (width > 1) {
          const int parents = (width + 1) >> 1;
          if ((node ^ 1) < width) {
            unsigned long long* slot =
                slots + ((size_t)(base + (node >> 1)) * gridDim.x + blockIdx.x) * kTileElems + e;
            const unsigned long long mine = (1ull << 32) | __float_as_uint(s);
            const unsigned long long old = __hip_atomic_exchange(
                slot, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((old >> 32) == 0) {   // first of the two: the sibling carries on
              carry = false;
              break;
            }
            const float other = __uint_as_float((unsigned)old);
            s = (node & 1) ? other + s : s + other;   // left + right
            __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          base += parents;
          node >>= 1;
          width = parents;
        }
        if (carry) *d = epilogue_apply(ep, s, d, n);
      }
    }
  }
}

// Slices: enough workgroups for every CU (or `target` slices if given), each
// slice at least one super-block.
// Exchange-tree nodes above the leaves for `slices` slices: the slot groups
// the in-kernel sum uses (one per node, a node without a right child included).
inline int tree_nodes(int slices) {
  int total = 0;
  for (int width = slices; width > 1; width = (width + 1) >> 1) total += (width + 1) >> 1;
  return total;
}

template <int CG, bool XCH = false>
SkinnyPlan plan_tile(const Problem& p, int target) {
  SkinnyPlan pl{};
  pl.strips = (p.N + CG * kGroupCols - 1) / (CG * kGroupCols);
  const int nsb = p.K / 16;
  int slices = target > 0 ? target : (256 + pl.strips - 1) / pl.strips;
  if (slices > nsb) slices = nsb;
  if (slices < 1) slices = 1;
  const int per = nsb > 0 ? (nsb + slices - 1) / slices : 0;
  pl.kslice = per;                                   // super-blocks per slice
  pl.splits = per > 0 ? (nsb + per - 1) / per : 1;   // no empty slice
  pl.partial_floats = (pl.splits > 1 && !XCH) ? (size_t)pl.splits * p.M * p.N : 0;
  pl.slot_words = (pl.splits > 1 && XCH)
                      ? (size_t)tree_nodes(pl.splits) * pl.strips * (CG * 2 * 4 * 64) : 0;
  pl.lds_bytes = 0;
  return pl;
}

template <int NW, int CG, int U, bool VA, bool VB, bool TA, bool XCH = false>
hipError_t launch_tile(const Problem& p, const SkinnyPlan& pl, float* partials,
                       const Epilogue& e, hipStream_t s) {
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.batch != 1)
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !(XCH ? (void*)pl.slots : (void*)partials)) return hipErrorInvalidValue;
  Problem pp = p;
  int per = pl.kslice, slices = pl.splits;
  float* part = partials;
  unsigned long long* sl = pl.slots;
  Epilogue ee = e;
  void* args[] = {&pp, &per, &slices, &part, &sl, &ee};
  hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_tile_kernel<NW, CG, U, VA, VB, TA, XCH>),
      dim3(pl.strips, pl.splits), dim3(NW * 64), args, 0, s);
  if (err != hipSuccess || pl.splits == 1 || XCH) return err;
  return launch_combine(p, slices, partials, s, e);
}

#define GEMMF32_SKINNY_TILE(NW, CG, U, S)                                                   \
  {"skinny_w" #NW "_c" #CG "_u" #U "_s" #S "_vec", 16, NW, U, true, true, S, false, false,  \
   &plan_tile<CG>, &launch_tile<NW, CG, U, true, true, false>},                             \
  {"skinny_w" #NW "_c" #CG "_u" #U "_s" #S "_veca", 16, NW, U, true, false, S, false, false, \
   &plan_tile<CG>, &launch_tile<NW, CG, U, true, false, false>},                            \
  {"skinny_w" #NW "_c" #CG "_u" #U "_s" #S "_vecb", 16, NW, U, false, true, S, false, false, \
   &plan_tile<CG>, &launch_tile<NW, CG, U, false, true, false>},                            \
  {"skinny_w" #NW "_c" #CG "_u" #U "_s" #S "_scalar", 16, NW, U, false, false, S, false,     \
   false, &plan_tile<CG>, &launch_tile<NW, CG, U, false, false, false>}
// A stored transposed (K x M), B as is
#define GEMMF32_SKINNY_TILE_TA(NW, CG, U, S)                                                \
  {"skinny_w" #NW "_c" #CG "_u" #U "_s" #S "_tn", 16, NW, U, false, true, S, true, false,   \
   &plan_tile<CG>, &launch_tile<NW, CG, U, false, true, true>}

// K slices added in-kernel through exchange slots (prefix skinnyx_); _vec
// takes any 4-byte aligned operands, _scalar is its 32-bit-load twin
#define GEMMF32_SKINNY_TILE_X1(NW, CG, U, S)                                                 \
  {"skinnyx_w" #NW "_c" #CG "_u" #U "_s" #S "_vec", 16, NW, U, true, true, S, false, false,  \
   &plan_tile<CG, true>, &launch_tile<NW, CG, U, true, true, false, true>}
#define GEMMF32_SKINNY_TILE_XS(NW, CG, U, S)                                                 \
  {"skinnyx_w" #NW "_c" #CG "_u" #U "_s" #S "_scalar", 16, NW, U, false, false, S, false,     \
   false, &plan_tile<CG, true>, &launch_tile<NW, CG, U, false, false, false, true>}
#define GEMMF32_SKINNY_TILE_X(NW, CG, U, S) \
  GEMMF32_SKINNY_TILE_X1(NW, CG, U, S), GEMMF32_SKINNY_TILE_XS(NW, CG, U, S)

#define GEMMF32_SKINNY_TILE_X_TA(NW, CG, U, S)                                               \
  {"skinnyx_w" #NW "_c" #CG "_u" #U "_s" #S "_tn", 16, NW, U, false, true, S, true, false,    \
   &plan_tile<CG, true>, &launch_tile<NW, CG, U, false, true, true, true>}

// Name: skinny_w<waves>_c<column groups of 32>_u<super-blocks in flight>_s<K
// slices, 0 = from the shape>_<load widths>, or _tn for A stored transposed;
// skinnyx_ for the in-kernel sum of the slices.
// The default build holds the kernels the tuning tables can pick; a build
// with GEMM_F32_SWEEP also holds the ones tuning sweeps compared them with.
const SkinnyVariant kVariants[] = {
    // 64-column strips, two super-blocks in flight per wave (32 KiB of B per
    // workgroup): 8 x 8192 x 8192 in 45 us against 48 us with the combine
    GEMMF32_SKINNY_TILE_X1(8, 2, 2, 0),
    GEMMF32_SKINNY_TILE_X_TA(8, 2, 2, 0),
    GEMMF32_SKINNY_TILE_X1(16, 2, 2, 0),
#if GEMM_F32_SWEEP
    GEMMF32_SKINNY_TILE_XS(8, 2, 2, 0),
    GEMMF32_SKINNY_TILE_XS(16, 2, 2, 0),
    GEMMF32_SKINNY_TILE(16, 1, 4, 1),    // 32 columns, all of K: no partial sums
    GEMMF32_SKINNY_TILE(8, 1, 4, 1),
    GEMMF32_SKINNY_TILE(16, 4, 4, 0),    // 128 columns, K split to fill the GPU
    GEMMF32_SKINNY_TILE(8, 4, 4, 0),
    GEMMF32_SKINNY_TILE(16, 2, 4, 0),    // 64 columns
    GEMMF32_SKINNY_TILE(8, 8, 4, 0),     // 256 columns
    GEMMF32_SKINNY_TILE(8, 4, 4, 2),
    GEMMF32_SKINNY_TILE(8, 2, 4, 0),
    GEMMF32_SKINNY_TILE(4, 4, 4, 0),
    GEMMF32_SKINNY_TILE(16, 8, 4, 0),
    GEMMF32_SKINNY_TILE(8, 4, 8, 0),     // 8 super-blocks in flight per wave
    GEMMF32_SKINNY_TILE(8, 4, 6, 0),
    GEMMF32_SKINNY_TILE(8, 8, 8, 0),
    GEMMF32_SKINNY_TILE(8, 4, 4, 8),     // 8 K slices: two workgroups per CU
    GEMMF32_SKINNY_TILE(8, 4, 8, 8),
    GEMMF32_SKINNY_TILE_TA(8, 4, 4, 0),
    GEMMF32_SKINNY_TILE_X(8, 2, 1, 0),
    GEMMF32_SKINNY_TILE_X(8, 2, 3, 0),
    GEMMF32_SKINNY_TILE_X(8, 2, 4, 0),
    GEMMF32_SKINNY_TILE_X(8, 4, 2, 0),
    GEMMF32_SKINNY_TILE_X(8, 4, 4, 0),
#endif
};

}  // namespace

int skinny_variant_count() {
  return (int)(sizeof(kVariants) / sizeof(kVariants[0])) + skinny_t_variant_count() +
         skinny_rows_variant_count() + skinny_tm_variant_count();
}
const SkinnyVariant& skinny_variant(int i) {
  const int n = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
  if (i < n) return kVariants[i];
  i -= n;
  if (i < skinny_t_variant_count()) return skinny_t_variant(i);
  i -= skinny_t_variant_count();
  if (i < skinny_rows_variant_count()) return skinny_rows_variant(i);
  return skinny_tm_variant(i - skinny_rows_variant_count());
}

}  // namespace gemmf32
