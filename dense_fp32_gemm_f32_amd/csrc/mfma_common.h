// Pieces shared by the two macro-tiled fp32 MFMA kernels of this library
// (global loads through registers, and direct-to-LDS loads): the workgroup
// to tile order, the tile configuration and the LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_f32_internal.h"

namespace gemmf32 {
namespace mfma {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// 16 bytes from a float address that is only 4-byte aligned.  Multi-dword
// global loads on gfx950 need dword alignment only, and the compiler emits one
// global_load_dwordx4 for this copy, so rows with any pitch load at 128 bits.
__device__ __forceinline__ float4 load4(const float* p) {
  float4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

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

template <int BM, int BN, int BK, int WM, int WN>
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
  static_assert(BN % 64 == 0, "the B swizzle needs 64-wide tile rows");
  static_assert(BK == 8 || BK == 16 || BK == 32 || BK == 64, "BK in {8, 16, 32, 64}");
  static_assert((BM * BK / 4) % kThreads == 0 && (BK * BN / 4) % kThreads == 0,
                "tile loads divide evenly over the threads");
  static constexpr int kLdsA = BM * BK;   // [m][k], k contiguous, 16-byte chunks swizzled
  static constexpr int kLdsB = BK * BN;   // [k][n], n contiguous, swizzled
};

// A tile in LDS: row m holds BK floats as kChunks 16-byte chunks; logical
// chunk c of row m sits at chunk c ^ swz_a(m).  Sixteen consecutive rows with
// the same logical chunk then cover all 64 banks, so both the 128-bit
// fragment reads (one row per lane) and the 128-bit tile writes are free of
// bank conflicts.
template <int kChunks>
__device__ __forceinline__ int swz_a(int m) {
  return (m / (16 / kChunks)) % kChunks;
}
// B tile in LDS: n of row k is XORed with 32 when bit 2 of k is set, so the
// rows k and k + 4 read together by one fragment land in opposite bank halves.
__device__ __forceinline__ int swz_b(int k) { return ((k >> 2) & 1) << 5; }

// Masked store of a wave's accumulator blocks (32 x 32 each, block (i, j) at
// rows row0 + 32 i, columns col0 + 32 j of C) with the update `ep`: register
// r of lane l is element (8 (r / 4) + 4 (l / 32) + r % 4, l % 32) of its block.
// raw: a K slice's partial sum, stored as is (the combine applies the update).
// The plain product (alpha 1, beta 0, no bias, identity) stores the sums
// directly, which is what the update computes for it (1 * s == s); the branch
// is uniform, so each store loop is free of per-element tests of the update.
template <int KFM, int KFN>
__device__ __forceinline__ void store_blocks(const floatx16 (&acc)[KFM][KFN], float* C,
                                             int64_t ldc, int M, int N, int row0, int col0,
                                             int lane, bool raw, const Epilogue& ep) {
  const int lr = lane & 31, lk = lane >> 5;
  const bool direct = raw || (ep.alpha == 1.f && ep.beta == 0.f && !ep.bias && ep.act == 0);
#pragma unroll
  for (int i = 0; i < KFM; ++i) {
#pragma unroll
    for (int j = 0; j < KFN; ++j) {
      const int col = col0 + 32 * j + lr;
      const int rbase = row0 + 32 * i + 4 * lk;
      if (col < N) {
        if (direct) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + 8 * (r >> 2) + (r & 3);
            if (row < M) C[(int64_t)row * ldc + col] = acc[i][j][r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + 8 * (r >> 2) + (r & 3);
            if (row < M) {
              float* c = C + (int64_t)row * ldc + col;
              *c = epilogue_apply(ep, acc[i][j][r], c, col);
            }
          }
        }
      }
    }
  }
}

// MFMA k-slot assignment.  One ds_read_b128 gives lane l four consecutive k
// of its A row: k = 8q + 4*(l/32) + s for s = 0..3.  MFMA step s therefore
// multiplies, in k-slot h = l/32, the term k = 8q + 4h + s; the B fragment of
// step s supplies B[8q + 4h + s][n] in the same slot.  Each k of the 8-wide
// group is used exactly once, so the sum is the same dot product.

}  // namespace mfma
}  // namespace gemmf32
