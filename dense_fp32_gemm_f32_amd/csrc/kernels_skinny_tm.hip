// Skinny-M fp32 GEMM with B stored transposed (N x K) on the matrix cores:
// C = alpha * op(A) B + beta * C for M <= 16.
//
// Element (m, j) of the product is row m of op(A) dotted with row j of the
// stored B^T.  At M = 16 every element of B feeds 16 multiply-adds, so at the
// HBM rate the vector ALUs (without packed math) would spend most of their
// issue slots on the dot products; v_mfma_f32_16x16x4_f32 does them instead,
// with the bound left at HBM.  Operand layout (wave64), for a block of 16 k
// starting at k0 and a group of 16 columns j0 .. j0 + 15:
//   A operand, lane l: op(A)[l % 16][k0 + 4 (l / 16) + s]      (step s = 0..3)
//   B operand, lane l: B^T[j0 + l % 16][k0 + 4 (l / 16) + s]
//   accumulator register r of lane l: C[4 (l / 16) + r][j0 + l % 16]
// so one 16-byte load per lane gives the four steps of a block: lanes l,
// l + 16, l + 32, l + 48 read 64 contiguous bytes of row j0 + l % 16, and
// each k of the block is used exactly once.
//
// Three kernels share this layout and differ in how B^T reaches the lanes:
//  - skinny_tm_kernel: straight into registers, one 64-byte piece of each of
//    16 rows per load (any alignment of B^T);
//  - skinny_tl_kernel: each wave copies its own chunks of 16 rows into LDS
//    (global_load_lds_dwordx4; 16-byte aligned B^T);
//  - skinny_tc_kernel: a ring of 16-row chunks in LDS shared by the
//    workgroup, each copy one whole 1 KiB run of one row (long K).
//
// Work split (skinny_tm_kernel): a workgroup of W waves owns JG groups of 16
// columns; its waves take the 16-k blocks of the K range in turn (wave w:
// blocks w, w + W, ...), so at any time the workgroup reads neighbouring
// blocks of the same rows, U blocks in flight per wave.  In every kernel the
// waves' partial tiles are added in LDS in wave order -- the per-group
// partials and their fixed-order sum of "GPU compute shaders" (How it works;
// Pitfalls: a fixed group count and order give the same bits on every run).
// When the column groups alone leave the GPU short of waves, K is also split
// over workgroups; the slices then go through the workspace and the combine
// kernel, added in slice order.
#include <cstdint>
#include <type_traits>

#include "gemm_f32_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace gemmf32 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
// four floats at a 4-byte aligned address (multi-dword global loads need
// dword alignment only), as one 128-bit load
typedef float floatx4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kTargetWaves = 4096;   // 16 per CU

// mfma::load_lds16 with the non-temporal hint (nt): B^T is read once, so
// its lines need not stay in the caches.
__device__ __forceinline__ void load_lds16_nt(const float* g, float* lds_wave) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) float*)lds_wave));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_addr)
      : "memory");
}
template <bool NT>
__device__ __forceinline__ void copy16(const float* g, float* lds_wave) {
  if constexpr (NT) {
    load_lds16_nt(g, lds_wave);
  } else {
    mfma::load_lds16(g, lds_wave);
  }
}

template <int W, int JG, int U, bool TA>
__global__ void __launch_bounds__(W * 64)
    skinny_tm_kernel(Problem p, int kslice, int slices, float* __restrict__ part, Epilogue ep) {
  __shared__ __attribute__((aligned(16))) float red[W][JG][4][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int M = p.M, N = p.N, K = p.K;
  const int j_base = blockIdx.x * (16 * JG);
  const int slice = blockIdx.y;
  const int kb = slice * kslice;
  const int ke = slice == slices - 1 ? K : min(K, kb + kslice);
  const int c16 = lane & 15, ks = lane >> 4;

  // this lane's rows of B^T (columns past N read row N - 1; never stored)
  const float* brow[JG];
#pragma unroll
  for (int g = 0; g < JG; ++g)
    brow[g] = p.B + (int64_t)min(j_base + 16 * g + c16, N - 1) * p.ldb + 4 * ks;
  // this lane's row of op(A) (rows past M read row M - 1 and are zeroed)
  const bool m_ok = c16 < M;
  const int mm = m_ok ? c16 : M - 1;
  const int64_t a_ks = TA ? p.lda : 1;   // stride of k in A's storage
  const float* arow = (TA ? p.A + mm : p.A + (int64_t)mm * p.lda) + (int64_t)(4 * ks) * a_ks;

  floatx4 acc[JG];
#pragma unroll
  for (int g = 0; g < JG; ++g) acc[g] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Blk {
    floatx4 b[JG];
    floatx4 a;
  };
  // the full 16-k blocks of the slice: [0, nb); this wave takes wave, wave + W, ...
  const int nb = (ke - kb) >> 4;
  int next = wave;
  // block t's loads; a prefetch past the last block re-reads block `wave`
  // and is multiplied as exact zeros, so the loop has no branch
  auto load = [&](Blk& x) {
    const int t = next < nb ? next : wave;
    const int64_t k = kb + 16 * t;
#pragma unroll
    for (int g = 0; g < JG; ++g)
      x.b[g] = __builtin_nontemporal_load(reinterpret_cast<const floatx4_a4*>(brow[g] + k));
    if (TA) {
      const float* a = arow + k * a_ks;
      x.a = floatx4{a[0], a[a_ks], a[2 * a_ks], a[3 * a_ks]};
    } else {
      x.a = *reinterpret_cast<const floatx4_a4*>(arow + k);
    }
    next += W;
  };
  auto mfma_blk = [&](const Blk& x, bool valid) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float av = (valid && m_ok) ? x.a[s] : 0.f;
#pragma unroll
      for (int g = 0; g < JG; ++g) {
        const float bv = valid ? x.b[g][s] : 0.f;
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[g], 0, 0, 0);
      }
    }
  };

  if (wave < nb) {
    Blk x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(x[u]);
    for (int t0 = wave; t0 < nb; t0 += U * W) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mfma_blk(x[u], t0 + u * W < nb);
        load(x[u]);
        // keep the rotation in program order: the other U - 1 blocks stay in
        // flight while this one is multiplied
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the last K % 16 values of the range, element by element, on one wave
  if (kb + 16 * nb < ke && wave == nb % W) {
    const int k0 = kb + 16 * nb;
    Blk x;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = k0 + 4 * ks + s;
      const bool ok = k < ke;
      const int kk = (ok ? k : ke - 1) - 4 * ks;
#pragma unroll
      for (int g = 0; g < JG; ++g) x.b[g][s] = ok ? brow[g][kk] : 0.f;
      x.a[s] = ok ? arow[(int64_t)kk * a_ks] : 0.f;
    }
    mfma_blk(x, true);
  }

  // the waves' partial tiles, added in wave order
#pragma unroll
  for (int g = 0; g < JG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][g][r][lane] = acc[g][r];
  __syncthreads();
  for (int e = tid; e < JG * 4 * 64; e += W * 64) {
    const int g = e / 256, r = (e / 64) % 4, l = e % 64;
    const int m = 4 * (l >> 4) + r;
    const int j = j_base + 16 * g + (l & 15);
    if (m < M && j < N) {
      float s = red[0][g][r][l];
#pragma unroll
      for (int w = 1; w < W; ++w) s += red[w][g][r][l];
      if (slices == 1) {
        float* d = p.C + (int64_t)m * p.ldc + j;
        *d = epilogue_apply(ep, s, d, j);
      } else {
        part[((size_t)slice * M + m) * N + j] = s;
      }
    }
  }
}

// The same product with B^T read in row runs of CK floats (CK = 256: whole
// 1 KiB runs, 64 lanes x 16 bytes of one row per load; CK = 128 or 64:
// 512 or 256-byte runs, two or four rows per load); the 64-byte runs of the
// kernel above stream about a third slower.
// Each wave owns CK-k chunks c = wave, wave + W, ... of the workgroup's 16
// rows and copies a chunk straight into its own LDS buffers with
// global_load_lds_dwordx4; the MFMA operand layout is then read out of LDS.
// 16-byte unit u of row r sits at unit u ^ r of the row's run, so the 16 rows
// a fragment read touches (lanes l % 16) fall in different banks.  ADMA: A's
// chunk (its 16 rows, A stored M x K) is copied the same way instead of
// loaded into registers by the lanes that use it (which costs a 64-byte piece
// of 16 rows per load).  NB buffers per wave: the next chunk loads while this
// one is multiplied.  B must be 16-byte aligned with a pitch that is a
// multiple of 4 (and A too, with ADMA); the last K % CK values of a slice go
// through direct loads.
// ROT: workgroup g starts its walk along the rows W g chunks in (mod the
// chunk count), so that at any time the workgroups' windows of W chunks lie at
// different offsets of their rows; without it every workgroup reads the same
// offset of its rows at the same time (rows one pitch apart).  NT: B^T is
// copied with the non-temporal hint.  A kernel that streams B^T through the
// caches without it leaves them in a state that costs the next streaming
// kernel about 10 us at 16 x 8192 x 8192 (measured on a kernel timed right
// after another); with both, 16 x 8192 x 4096 takes 30.0 us against 34.3 us.
template <int W, int NB, int CK, bool ADMA, bool TA, bool ROT = false, bool NT = false>
__global__ void __launch_bounds__(W * 64)
    skinny_tl_kernel(Problem p, int kslice, int slices, float* __restrict__ part, Epilogue ep) {
  static_assert(NB == 1 || NB == 2, "one or two buffers per wave");
  static_assert(CK == 64 || CK == 128 || CK == 256, "256-byte, 512-byte or 1 KiB runs");
  static_assert(!(ADMA && TA), "copies of A need its rows along k");
  constexpr int kLoads = CK / 16;          // copies per matrix per chunk (1 KiB each)
  constexpr int kRowsPerLoad = 256 / CK;   // rows one copy covers
  constexpr int kBlocks = CK / 16;         // 16-k blocks per chunk
  constexpr int kMats = ADMA ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float lds[W][NB][kMats][16 * CK];
  __shared__ __attribute__((aligned(16))) float red[W][4][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int M = p.M, N = p.N, K = p.K;
  const int j_base = blockIdx.x * 16;
  const int slice = blockIdx.y;
  const int kb = slice * kslice;
  const int ke = slice == slices - 1 ? K : min(K, kb + kslice);
  const int c16 = lane & 15, ks = lane >> 4;

  // Copies: lane l of copy i lands at unit `pos` of row kRowsPerLoad i + rl of
  // the buffer, so it fetches unit pos ^ row of that row (rows of B^T past N
  // read row N - 1, rows of A past M row M - 1; neither is stored)
  const int rl = lane / (CK / 4);
  const int pos = lane % (CK / 4);
  const float* bsrc[kLoads];
  const float* asrc[ADMA ? kLoads : 1];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = kRowsPerLoad * i + rl;
    bsrc[i] = p.B + (int64_t)min(j_base + r, N - 1) * p.ldb + 4 * (pos ^ r);
    if (ADMA) asrc[i] = p.A + (int64_t)min(r, M - 1) * p.lda + 4 * (pos ^ r);
  }
  // this lane's row of op(A) for direct loads (rows past M read row M - 1 and
  // are zeroed)
  const bool m_ok = c16 < M;
  const int mm = m_ok ? c16 : M - 1;
  const int64_t a_ks = TA ? p.lda : 1;
  const float* arow = (TA ? p.A + mm : p.A + (int64_t)mm * p.lda) + (int64_t)(4 * ks) * a_ks;
  auto load_a = [&](int64_t k) -> floatx4 {
    const float* a = arow + k * a_ks;
    if (TA) return floatx4{a[0], a[a_ks], a[2 * a_ks], a[3 * a_ks]};
    return *reinterpret_cast<const floatx4_a4*>(a);
  };

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mfma4 = [&](floatx4 a, floatx4 b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float av = m_ok ? a[s] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b[s], acc, 0, 0, 0);
    }
  };

  // Whole CK-k chunks of the slice; this wave's are wave, wave + W, ...
  // Chunk i is issued as its operand loads of A (or A's copies), then B's
  // copies, into buffer i % NB; loads return in issue order, so waiting until
  // at most the next chunk's loads are outstanding completes chunk i.
  const int nc = (ke - kb) / CK;
  const int mine = wave < nc ? (nc - wave + W - 1) / W : 0;
  // chunk wave + i W of the slice is chunk (wave + i W + rot) mod nc: every
  // chunk still goes to exactly one wave
  const int rot = ROT && nc > 0 ? (int)(((int64_t)blockIdx.x * W) % nc) : 0;
  floatx4 a[NB][ADMA ? 1 : kBlocks];
  // chunk i into buffer B_ (= i % NB, a compile-time index of the registers)
  auto issue = [&](int i, auto buf_tag) {
    constexpr int B_ = decltype(buf_tag)::value;
    int c = wave + i * W + rot;
    if (ROT && c >= nc) c -= nc;
    const int64_t k0 = kb + CK * (int64_t)c;
    if constexpr (ADMA) {
#pragma unroll
      for (int c = 0; c < kLoads; ++c) mfma::load_lds16(asrc[c] + k0, &lds[wave][B_][1][c * 256]);
    } else {
#pragma unroll
      for (int q = 0; q < kBlocks; ++q) a[B_][q] = load_a(k0 + 16 * q);
    }
#pragma unroll
    for (int c = 0; c < kLoads; ++c) copy16<NT>(bsrc[c] + k0, &lds[wave][B_][0][c * 256]);
  };
  auto step = [&](int i, auto buf_tag) {
    constexpr int B_ = decltype(buf_tag)::value;
    // memory instructions of one chunk: A's (copies, or operand loads, four
    // per block when A is stored transposed), then B's copies
    constexpr int kOps = (ADMA ? kLoads : (TA ? 4 : 1) * kBlocks) + kLoads;
    if (NB > 1 && kOps <= 63 && i + 1 < mine) {
      __builtin_amdgcn_s_waitcnt(0x0f70 | (kOps & 15) | ((kOps >> 4) << 14));   // vmcnt(kOps)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);                                       // vmcnt(0)
    }
    const float* brow = &lds[wave][B_][0][c16 * CK];
    const float* alds = &lds[wave][B_][ADMA ? 1 : 0][c16 * CK];
#pragma unroll
    for (int q = 0; q < kBlocks; ++q) {
      const int u = (4 * q + ks) ^ c16;
      const floatx4 bv = *reinterpret_cast<const floatx4*>(brow + 4 * u);
      if constexpr (ADMA) {
        mfma4(*reinterpret_cast<const floatx4*>(alds + 4 * u), bv);
      } else {
        mfma4(a[B_][q], bv);
      }
    }
    // the buffer is read before the copy of chunk i + NB overwrites it
    __builtin_amdgcn_s_waitcnt(0xc07f);                                          // lgkmcnt(0)
    if (i + NB < mine) issue(i + NB, buf_tag);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, NB - 1>;
  if (0 < mine) issue(0, B0{});
  if (NB > 1 && 1 < mine) issue(1, B1{});
  for (int i = 0; i < mine; i += NB) {
    step(i, B0{});
    if (NB > 1 && i + 1 < mine) step(i + 1, B1{});
  }
  __builtin_amdgcn_s_waitcnt(0);

  // the rest of the slice (K % CK values of the last one), direct loads
  const int k_rest = kb + CK * nc;
  if (k_rest < ke && wave == nc % W) {
    const float* brow = p.B + (int64_t)min(j_base + c16, N - 1) * p.ldb + 4 * ks;
    int k0 = k_rest;
    for (; k0 + 16 <= ke; k0 += 16)
      mfma4(load_a(k0), *reinterpret_cast<const floatx4_a4*>(brow + k0));
    if (k0 < ke) {
      floatx4 x, y;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = k0 + 4 * ks + s;
        const bool ok = k < ke;
        const int kk = (ok ? k : ke - 1) - 4 * ks;
        x[s] = ok ? arow[(int64_t)kk * a_ks] : 0.f;
        y[s] = ok ? brow[kk] : 0.f;
      }
      mfma4(x, y);
    }
  }

  // the waves' partial tiles, added in wave order
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  for (int e = tid; e < 4 * 64; e += W * 64) {
    const int r = e / 64, l = e % 64;
    const int m = 4 * (l >> 4) + r;
    const int j = j_base + (l & 15);
    if (m < M && j < N) {
      float s = red[0][r][l];
#pragma unroll
      for (int w = 1; w < W; ++w) s += red[w][r][l];
      if (slices == 1) {
        float* d = p.C + (int64_t)m * p.ldc + j;
        *d = epilogue_apply(ep, s, d, j);
      } else {
        part[((size_t)slice * M + m) * N + j] = s;
      }
    }
  }
}

// The same product with the workgroup's 16 rows of B^T streamed through a
// ring of NBUF chunk buffers shared by all its waves.  A chunk is 256 k of the
// 16 rows (16 KiB); each of its 16 copies into LDS is one whole 1 KiB run of
// one row (64 lanes x 16 bytes, non-temporal), and NBUF - 1 chunks are in
// flight while the waves multiply the one that has landed.  Few bytes in
// flight stream best here: two buffers (one chunk in flight, 32 KiB per CU at
// two workgroups per CU) take 49.8 us at 16 x 8192 x 8192 with 16 waves,
// three buffers 55.2 us and four 55.8 us.  Wave w multiplies 16-k blocks
// w, w + W, ... of every chunk, so the multiply-adds of a chunk are spread
// over the SIMDs rather than waiting on one wave.  One barrier per chunk: after it the chunk is in LDS and every
// wave is done with the previous one, whose buffer then takes the copies of
// chunk t + NBUF - 1.  The copies of row r fetch 16-byte unit l ^ r for lane
// l (the swizzle of the kernel above), and the operand of op(A) for a block
// goes to registers when its chunk is issued.  Each wave's partial tile is
// added in wave order at the end (a fixed order, so reruns give the same
// bits).  Workgroup g walks its chunks starting at chunk g (mod the count),
// so that the workgroups read different offsets of their rows.
template <int N_, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N_, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N_>(f, std::make_integer_sequence<int, N_>{});
}
template <int N_>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N_ >= 0 && N_ <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N_ & 15) | ((N_ >> 4) << 14));
}

template <int W, int NBUF, bool TA>
__global__ void __launch_bounds__(W * 64)
    skinny_tc_kernel(Problem p, int kslice, int slices, float* __restrict__ part, Epilogue ep) {
  static_assert(W == 4 || W == 8 || W == 16, "16 rows per chunk: 16 / W copies per wave");
  static_assert(NBUF >= 2 && NBUF <= 8, "ring depth");
  constexpr int CK = 256;                               // k per chunk
  constexpr int kCopies = 16 / W;                       // 1 KiB copies per wave and chunk
  constexpr int kBlocks = 16 / W;                       // 16-k blocks per wave and chunk
  constexpr int kOps = kCopies + (TA ? 4 : 1) * kBlocks;  // memory instructions per chunk
  static_assert((NBUF - 2) * kOps <= 63, "chunks in flight beyond the vmcnt range");
  static_assert(W * 4 * 64 <= NBUF * 16 * CK, "the partial tiles reuse the ring");
  __shared__ __attribute__((aligned(16))) float ring[NBUF][16 * CK];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int M = p.M, N = p.N, K = p.K;
  const int j_base = blockIdx.x * 16;
  const int slice = blockIdx.y;
  const int kb = slice * kslice;
  const int ke = slice == slices - 1 ? K : min(K, kb + kslice);
  const int c16 = lane & 15, ks = lane >> 4;

  // copy c of a chunk is row r = wave + W c (rows past N read row N - 1 and
  // are not stored); lane l lands at unit l of the row's run in LDS
  const float* bsrc[kCopies];
#pragma unroll
  for (int c = 0; c < kCopies; ++c) {
    const int r = wave + W * c;
    bsrc[c] = p.B + (int64_t)min(j_base + r, N - 1) * p.ldb + 4 * (lane ^ r);
  }
  // this lane's row of op(A) (rows past M read row M - 1 and are zeroed)
  const bool m_ok = c16 < M;
  const int mm = m_ok ? c16 : M - 1;
  const int64_t a_ks = TA ? p.lda : 1;
  const float* arow = (TA ? p.A + mm : p.A + (int64_t)mm * p.lda) + (int64_t)(4 * ks) * a_ks;
  auto load_a = [&](int64_t k) -> floatx4 {
    const float* a = arow + k * a_ks;
    if (TA) return floatx4{a[0], a[a_ks], a[2 * a_ks], a[3 * a_ks]};
    return *reinterpret_cast<const floatx4_a4*>(a);
  };
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mfma4 = [&](floatx4 a, floatx4 b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float av = m_ok ? a[s] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b[s], acc, 0, 0, 0);
    }
  };

  const int nc = (ke - kb) / CK;
  const int rot = nc > 0 ? (int)(blockIdx.x % (unsigned)nc) : 0;
  floatx4 areg[NBUF][kBlocks];
  // chunk t into ring slot S (= t % NBUF, a compile-time index of areg)
  auto issue = [&](int t, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    int ci = t + rot;
    if (ci >= nc) ci -= nc;
    const int64_t k0 = kb + (int64_t)CK * ci;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) areg[S][b] = load_a(k0 + 16 * (wave + W * b));
#pragma unroll
    for (int c = 0; c < kCopies; ++c) load_lds16_nt(bsrc[c] + k0, &ring[S][(wave + W * c) * CK]);
  };
  auto step = [&](int t, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    // chunk t has landed when at most the chunks issued after it are
    // outstanding (loads complete in issue order)
    const int later = min(NBUF - 2, nc - 1 - t);
    static_for<NBUF - 1>([&](auto J) {
      if (later == decltype(J)::value) wait_vmcnt<decltype(J)::value * kOps>();
    });
    __syncthreads();
    if (t + NBUF - 1 < nc) issue(t + NBUF - 1, std::integral_constant<int, (S + NBUF - 1) % NBUF>{});
    const float* brow = &ring[S][c16 * CK];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const int u = (4 * (wave + W * b) + ks) ^ c16;
      mfma4(areg[S][b], *reinterpret_cast<const floatx4*>(brow + 4 * u));
    }
  };
  static_for<NBUF - 1>([&](auto I) {
    if (decltype(I)::value < nc) issue(decltype(I)::value, I);
  });
  for (int t0 = 0; t0 < nc; t0 += NBUF) {
    static_for<NBUF>([&](auto I) {
      if (t0 + decltype(I)::value < nc) step(t0 + decltype(I)::value, I);
    });
  }

  // the rest of the slice (K % 256 values of the last one): 16-k blocks over
  // the waves, then the partial block, with direct loads
  const int k_rest = kb + CK * nc;
  if (k_rest < ke) {
    const float* brow = p.B + (int64_t)min(j_base + c16, N - 1) * p.ldb + 4 * ks;
    const int nfull = (ke - k_rest) / 16;
    for (int q = wave; q < nfull; q += W) {
      const int k0 = k_rest + 16 * q;
      mfma4(load_a(k0), *reinterpret_cast<const floatx4_a4*>(brow + k0));
    }
    const int k0 = k_rest + 16 * nfull;
    if (k0 < ke && wave == nfull % W) {
      floatx4 x, y;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = k0 + 4 * ks + s;
        const bool ok = k < ke;
        const int kk = (ok ? k : ke - 1) - 4 * ks;
        x[s] = ok ? arow[(int64_t)kk * a_ks] : 0.f;
        y[s] = ok ? brow[kk] : 0.f;
      }
      mfma4(x, y);
    }
  }

  // the waves' partial tiles, added in wave order (in the ring's memory, once
  // every wave is done with it)
  __syncthreads();
  float* red = &ring[0][0];
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  for (int e = tid; e < 4 * 64; e += W * 64) {
    const int r = e / 64, l = e % 64;
    const int m = 4 * (l >> 4) + r;
    const int j = j_base + (l & 15);
    if (m < M && j < N) {
      float s = red[r * 64 + l];
#pragma unroll
      for (int w = 1; w < W; ++w) s += red[(w * 4 + r) * 64 + l];
      if (slices == 1) {
        float* d = p.C + (int64_t)m * p.ldc + j;
        *d = epilogue_apply(ep, s, d, j);
      } else {
        part[((size_t)slice * M + m) * N + j] = s;
      }
    }
  }
}

// K slices only when the column groups alone give too few waves; each slice
// at least 4 blocks per wave.
template <int W, int JG>
SkinnyPlan plan_tm(const Problem& p, int target) {
  SkinnyPlan pl{};
  pl.strips = (p.N + 16 * JG - 1) / (16 * JG);
  const int64_t nb = p.K / 16;
  int64_t slices = target > 0 ? target
                              : (kTargetWaves + (int64_t)pl.strips * W - 1) / ((int64_t)pl.strips * W);
  const int64_t cap = nb / (4 * W) > 1 ? nb / (4 * W) : 1;
  if (slices > cap) slices = cap;
  if (slices < 1) slices = 1;
  const int64_t per = nb > 0 ? (nb + slices - 1) / slices : 0;   // blocks per slice
  pl.splits = per > 0 ? (int)((nb + per - 1) / per) : 1;         // no empty slice
  pl.kslice = per > 0 ? (int)(16 * per) : p.K;
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.lds_bytes = 0;
  return pl;
}

template <int W, int JG, int U, bool TA>
hipError_t launch_tm(const Problem& p, const SkinnyPlan& pl, float* partials, const Epilogue& e,
                     hipStream_t s) {
  // every slice non-empty: slice s covers [s * kslice, ...), the last to K
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.M > 16 || p.batch != 1 ||
      pl.kslice <= 0 || (int64_t)pl.kslice * (pl.splits - 1) >= p.K)
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !partials) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, slices = pl.splits;
  float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &kslice, &slices, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_tm_kernel<W, JG, U, TA>),
      dim3(pl.strips, pl.splits), dim3(W * 64), args, 0, s);
  if (err != hipSuccess || pl.splits == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

template <int W, int CK>
SkinnyPlan plan_tl(const Problem& p, int target) {
  SkinnyPlan pl{};
  pl.strips = (p.N + 15) / 16;
  const int64_t nc = p.K / CK;
  int64_t slices = target > 0 ? target
                              : (kTargetWaves + (int64_t)pl.strips * W - 1) / ((int64_t)pl.strips * W);
  const int64_t cap = nc / (2 * W) > 1 ? nc / (2 * W) : 1;   // at least 2 chunks per wave
  if (slices > cap) slices = cap;
  if (slices < 1) slices = 1;
  const int64_t per = nc > 0 ? (nc + slices - 1) / slices : 0;   // chunks per slice
  pl.splits = per > 0 ? (int)((nc + per - 1) / per) : 1;
  pl.kslice = per > 0 ? (int)(CK * per) : p.K;
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.lds_bytes = 0;
  return pl;
}

// K slices only when the column groups alone give fewer than two workgroups
// per CU (the ring keeps one workgroup's memory traffic going with few
// waves); each slice at least 2 NBUF chunks.
template <int W, int NBUF>
SkinnyPlan plan_tc(const Problem& p, int target) {
  SkinnyPlan pl{};
  pl.strips = (p.N + 15) / 16;
  const int64_t nc = p.K / 256;
  constexpr int64_t kTargetGroups = 512;
  int64_t slices = target > 0 ? target : (kTargetGroups + pl.strips - 1) / pl.strips;
  const int64_t cap = nc / (2 * NBUF) > 1 ? nc / (2 * NBUF) : 1;
  if (slices > cap) slices = cap;
  if (slices < 1) slices = 1;
  const int64_t per = nc > 0 ? (nc + slices - 1) / slices : 0;   // chunks per slice
  pl.splits = per > 0 ? (int)((nc + per - 1) / per) : 1;
  pl.kslice = per > 0 ? (int)(256 * per) : p.K;
  pl.partial_floats = pl.splits > 1 ? (size_t)pl.splits * p.M * p.N : 0;
  pl.lds_bytes = 0;
  return pl;
}

template <int W, int NBUF, bool TA>
hipError_t launch_tc(const Problem& p, const SkinnyPlan& pl, float* partials, const Epilogue& e,
                     hipStream_t s) {
  // the copies into LDS need 16-byte aligned rows of B^T
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.M > 16 || p.batch != 1 ||
      pl.kslice <= 0 || (int64_t)pl.kslice * (pl.splits - 1) >= p.K || p.ldb % 4 != 0 ||
      (reinterpret_cast<uintptr_t>(p.B) & 15) != 0)
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !partials) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, slices = pl.splits;
  float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &kslice, &slices, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_tc_kernel<W, NBUF, TA>), dim3(pl.strips, pl.splits),
      dim3(W * 64), args, 0, s);
  if (err != hipSuccess || pl.splits == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

template <int W, int NB, int CK, bool ADMA, bool TA, bool ROT = false, bool NT = false>
hipError_t launch_tl(const Problem& p, const SkinnyPlan& pl, float* partials, const Epilogue& e,
                     hipStream_t s) {
  // the copies into LDS need 16-byte aligned rows of B^T
  if (pl.strips <= 0 || pl.splits < 1 || pl.splits > 65535 || p.M > 16 || p.batch != 1 ||
      pl.kslice <= 0 || (int64_t)pl.kslice * (pl.splits - 1) >= p.K || p.ldb % 4 != 0 ||
      (reinterpret_cast<uintptr_t>(p.B) & 15) != 0 ||
      (ADMA && (p.lda % 4 != 0 || (reinterpret_cast<uintptr_t>(p.A) & 15) != 0)))
    return hipErrorInvalidConfiguration;
  if (pl.splits > 1 && !partials) return hipErrorInvalidValue;
  Problem pp = p;
  int kslice = pl.kslice, slices = pl.splits;
  float* part = partials;
  Epilogue ee = e;
  void* args[] = {&pp, &kslice, &slices, &part, &ee};
  const hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_tl_kernel<W, NB, CK, ADMA, TA, ROT, NT>), dim3(pl.strips, pl.splits),
      dim3(W * 64), args, 0, s);
  if (err != hipSuccess || pl.splits == 1) return err;
  return launch_combine(p, slices, partials, s, e);
}

// Name: skinnytm_w<waves>_j<16-column groups>_u<blocks in flight>_<nt|tt>.
#define GEMMF32_SKINNY_TM(W, JG, U)                                                        \
  {"skinnytm_w" #W "_j" #JG "_u" #U "_nt", 16, W, U, true, true, 0, false, true,          \
   &plan_tm<W, JG>, &launch_tm<W, JG, U, false>},                                          \
  {"skinnytm_w" #W "_j" #JG "_u" #U "_tt", 16, W, U, false, true, 0, true, true,          \
   &plan_tm<W, JG>, &launch_tm<W, JG, U, true>}

// Name: skinnytl_w<waves>_b<LDS buffers per wave>_k<CK>[_a|_p]_<nt|tt> (_a:
// A's chunks copied into LDS too; _p: the plain walk, every workgroup from
// chunk 0, through the caches); needs B 16-byte aligned with a pitch that is
// a multiple of 4 (b16), and A too with _a.  The others start workgroup g's
// walk W g chunks in and copy B^T with the non-temporal hint.
#define GEMMF32_SKINNY_TL(W, NB, CK)                                                          \
  {"skinnytl_w" #W "_b" #NB "_k" #CK "_nt", 16, W, NB, true, true, 0, false, true,           \
   &plan_tl<W, CK>, &launch_tl<W, NB, CK, false, false, true, true>, true},                    \
  {"skinnytl_w" #W "_b" #NB "_k" #CK "_tt", 16, W, NB, false, true, 0, true, true,           \
   &plan_tl<W, CK>, &launch_tl<W, NB, CK, false, true, true, true>, true}
#define GEMMF32_SKINNY_TL_P(W, NB, CK)                                                        \
  {"skinnytl_w" #W "_b" #NB "_k" #CK "_p_nt", 16, W, NB, true, true, 0, false, true,         \
   &plan_tl<W, CK>, &launch_tl<W, NB, CK, false, false, false, false>, true},                  \
  {"skinnytl_w" #W "_b" #NB "_k" #CK "_p_tt", 16, W, NB, false, true, 0, true, true,         \
   &plan_tl<W, CK>, &launch_tl<W, NB, CK, false, true, false, false>, true}
#define GEMMF32_SKINNY_TL_A(W, NB, CK)                                                        \
  {"skinnytl_w" #W "_b" #NB "_k" #CK "_a_nt", 16, W, NB, true, true, 0, false, true,         \
   &plan_tl<W, CK>, &launch_tl<W, NB, CK, true, false, true, true>, true, true}

// Name: skinnytc_w<waves>_n<ring buffers>_<nt|tt>; needs B 16-byte aligned
// with a pitch that is a multiple of 4 (b16).
#define GEMMF32_SKINNY_TC(W, NBUF)                                                            \
  {"skinnytc_w" #W "_n" #NBUF "_nt", 16, W, NBUF, true, true, 0, false, true,                \
   &plan_tc<W, NBUF>, &launch_tc<W, NBUF, false>, true},                                      \
  {"skinnytc_w" #W "_n" #NBUF "_tt", 16, W, NBUF, false, true, 0, true, true,                \
   &plan_tc<W, NBUF>, &launch_tc<W, NBUF, true>, true}

// The default build holds the kernels the tuning table picks; a build with
// GEMM_F32_SWEEP also holds the ones tuning sweeps compared them with.
const SkinnyVariant kTmVariants[] = {
    // K >= 8192: the shared ring with one 16 KiB chunk in flight per
    // workgroup (16 x 8192 x 8192 with B^T: 45.0 us against 62.6 us for the
    // per-wave copies, same box, each timed after a call of itself)
    GEMMF32_SKINNY_TC(8, 2),
    GEMMF32_SKINNY_TC(16, 2),
    // shorter K: per-wave copies in 256-byte runs, 16 waves, one buffer each
    // (two workgroups per CU, 64 KiB of LDS each; 16 x 8192 x 4096: 30.0 us
    // against 53.2 us for the ring)
    GEMMF32_SKINNY_TL(16, 1, 64),
    // any alignment of B^T: 64-byte runs
    GEMMF32_SKINNY_TM(8, 1, 4),
#if GEMM_F32_SWEEP
    GEMMF32_SKINNY_TC(4, 2),
    GEMMF32_SKINNY_TC(4, 3),
    GEMMF32_SKINNY_TC(16, 3),
    GEMMF32_SKINNY_TC(16, 4),
    GEMMF32_SKINNY_TL_P(16, 1, 64),
    GEMMF32_SKINNY_TL(8, 1, 256),
    GEMMF32_SKINNY_TL(8, 2, 128),
    GEMMF32_SKINNY_TL(16, 1, 128),
    GEMMF32_SKINNY_TL(16, 2, 64),
    GEMMF32_SKINNY_TL_A(8, 1, 128),
    GEMMF32_SKINNY_TL_A(16, 1, 64),
    GEMMF32_SKINNY_TL_A(8, 2, 64),
    GEMMF32_SKINNY_TM(8, 2, 4),
    GEMMF32_SKINNY_TM(4, 2, 4),
    GEMMF32_SKINNY_TM(8, 4, 2),
    GEMMF32_SKINNY_TM(8, 1, 8),
    GEMMF32_SKINNY_TM(4, 4, 4),
#endif
};

}  // namespace

int skinny_tm_variant_count() { return (int)(sizeof(kTmVariants) / sizeof(kTmVariants[0])); }
const SkinnyVariant& skinny_tm_variant(int i) { return kTmVariants[i]; }

}  // namespace gemmf32
