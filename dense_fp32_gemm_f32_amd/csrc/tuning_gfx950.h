// Tuning table for gfx950 (MI355X): which kernel gemm_f32 runs for a shape.
//
// The first row whose bounds hold and whose kernel can take the arguments
// wins.  At each size the kernels with direct-to-LDS loads (16-byte aligned A
// and B, lda, ldb and N multiples of 4, K a multiple of the K-tile) come
// first, then the register-staged kernels that take any 4-byte aligned
// operands.  The choices are the fastest measured per shape class with
// dense_fp32_gemm_f32_amd/tune.py.
//
// Columns:
//   max_m        the row applies when M <= max_m
//   min_tiles    ... and the grid of 128 x 128 tiles has at least this many tiles
//   kernel       a name in the kernel table
//   wave_slots   ... and (if not 0) the kernel's own workgroups, wave_slots of
//                them resident per CU, fill their last wave of the 256 CUs to
//                at least 90 % or make 4 waves or more: a large tile is taken
//                only where it leaves no part-empty last wave
//   max_tiles    ... and (if not 0) the grid has at most this many tiles
#pragma once

#include <cstdint>

namespace gemmf32 {

constexpr int64_t kNumCus = 256;   // MI355X

struct TuningRow {
  int64_t max_m;
  int64_t min_tiles;
  const char* kernel;
  int wave_slots = 0;
  int64_t max_tiles = 0;
};

constexpr int64_t kAnyM = INT64_C(0x7fffffff);

constexpr TuningRow kTuningGfx950[] = {
    // wide skinny products (N above 20k): few K slices of 512-column strips
    // streamed in KiB row runs (8 x 28672 x 4096: 81 us against 92 us)
    {8, 160, "skinnyr_c2_r4_u4_m2x4_s0_nn"},
    // 64-column strips, K slices added in-kernel through exchange slots
    // (8 x 8192 x 8192: 45 us against 48 us for 128-column strips and a
    // combine dispatch; 8 x 512 x 8192: 13 us against 18 us).  Up to 2048
    // columns, 16 waves per workgroup keep more of B in flight (8 x 1024 x
    // 8192: 13.8 us against 15.2 us; 8 x 512 x 8192: 12.0 against 14.0 us)
    {16, 0, "skinnyx_w16_c2_u2_s0_vec", 0, 16},
    {16, 0, "skinnyx_w8_c2_u2_s0_vec"},
    // 256 x 256 tiles, 8 waves of 64 x 128 (4096^3: 939 us against 958 us)
    {kAnyM, 768, "mfma_256x256x32_w64x128_d6_vec", 1},
    {kAnyM, 768, "mfma_128x256x16_w64x128_d6_vec"},
    // operands the 16-byte direct loads cannot take (pitches or N not
    // multiples of 4, K not a multiple of the K-tile): 64 x 64 tiles copied
    // into LDS one float per lane (4095^3: 1030 us against 1063 us staged
    // through registers; 4096 x 4097 x 4096: 1070 us against 1158 us for the
    // best larger tile); then the register-staged tile whose grid fills its
    // waves (K below two K-tiles, or pitches beyond 32-bit tile offsets)
    {kAnyM, 768, "mfma_64x64x16_w32x32_d4_vec"},
    {kAnyM, 768, "mfma_128x128x32_w64x64_p5_vec", 2},
    // 128 x 192 or 192 x 128 tiles where one per CU makes whole waves
    // (2048 x 3072 x 1536: 148 us against 192 us for 128 x 128 tiles)
    {kAnyM, 192, "mfma_128x192x32_w32x96_d6_vec", 1},
    {kAnyM, 192, "mfma_192x128x32_w96x32_d6_vec", 1},
    // 128 x 128 tiles, 8 waves of 64 x 32 (2048^3: 133.5 us against 137.9 us
    // for 4 waves of 64 x 64, which remain for K a multiple of 16 only)
    {kAnyM, 192, "mfma_128x128x32_w64x32_d6_vec"},
    {kAnyM, 192, "mfma_128x128x16_w64x64_d6_vec"},
    // unaligned operands: single-float direct copies (2047 x 3001 x 1531:
    // 150.3 us against 166.0 us for the register-staged 128 x 192 tile;
    // 2048 x 2048 x 2047: 139.3 against 148.3 us), then 128 x 192 or 192 x
    // 128 register-staged tiles of 8 waves where they make whole waves
    {kAnyM, 192, "mfma_64x64x16_w32x32_d4_vec"},
    {kAnyM, 192, "mfma_128x192x32_w32x96_p5_vec", 1},
    {kAnyM, 192, "mfma_192x128x32_w96x32_p5_vec", 1},
    {kAnyM, 192, "mfma_64x64x32_w32x32_p5_vec"},
    {kAnyM, 24, "mfma_64x64x32_w32x32_d6_vec"},
    // unaligned: 1023 x 1025 x 1027 44.2 us against 49.1 us staged through
    // registers; 767 x 769 x 771 23.0 against 26.3 us
    {kAnyM, 24, "mfma_64x64x32_w32x32_d4_vec"},
    {kAnyM, 24, "mfma_64x64x32_w32x32_p5_vec"},
    // fewer than 24 tiles of 128 x 128 (512^3: 9.4 us against 12.9 us): 32 x 32
    // tiles, K split over 4 waves, fragments straight from global memory
    {kAnyM, 0, "mfma_32x32x8_k4_g4_small"},
};

// A transposed operand (any epilogue): the first row with at least min_tiles
// tiles of 128 x 128 whose kernel, with the layout suffix (_nt, _tn, _tt) of
// the call, takes the arguments (and, if wave_slots is not 0, fills whole
// waves as above).  Direct-to-LDS tiles come first; the register-staged tiles
// after them take any 4-byte aligned operands.  A and B as stored with an
// epilogue (alpha, beta, bias, activation) use the plain table above: its
// kernels apply the epilogue.
struct TuningRowEx {
  int64_t min_tiles;
  const char* kernel;
  int wave_slots = 0;
};
constexpr TuningRowEx kTuningGfx950Ex[] = {
    {768, "mfmaex_256x256x32_w64x128_d6", 1},
    {768, "mfmaex_128x128x32_w64x32_d6"},
    {768, "mfmaex_128x128x16_w64x64"},
    {192, "mfmaex_128x128x32_w64x32_d6"},
    {192, "mfmaex_128x64x32_w64x32"},
    {0, "mfmaex_64x64x32_w32x32_d6"},
    {0, "mfmaex_64x64x32_w32x32"},
};

// M <= 16 with a transposed operand or an epilogue: the first row whose max_m,
// layout (ta: A stored K x M, tb: B stored N x K) and max_n (if not 0) match.
struct TuningRowSkinny {
  int64_t max_m;
  bool ta, tb;
  const char* kernel;
  int64_t max_n = 0;   // 0: any N
  int64_t min_k = 0;   // 0: any K
};
constexpr TuningRowSkinny kTuningGfx950Skinny[] = {
    {16, false, false, "skinnyx_w16_c2_u2_s0_vec", 2048},
    {16, false, false, "skinnyx_w8_c2_u2_s0_vec"},
    {16, true, false, "skinnyx_w8_c2_u2_s0_tn"},
    // B stored N x K, 16-byte aligned rows: for K >= 8192 a ring of 16-row
    // chunks shared by the workgroup with one chunk in flight (16 x 8192 x
    // 8192: 45.0 us, A stored transposed 46.4 us); 8 waves for M <= 8 up to
    // N = 8192 (8 x 8192 x 8192 timed back to back: 46.2 against 48.7 us),
    // 16 waves otherwise (16 x 8192 x 8192: 49.0 against 49.6 us; 16 x
    // 16384 x 8192: 93.6 against 101.8 us); shorter K: each wave copies its
    // own chunks (16 x 8192 x 4096: 30.0 against 53.2 us).  B^T not 16-byte
    // aligned: the vector-ALU dot products for M <= 8, 64-byte runs on the
    // matrix cores above that.
    {8, false, true, "skinnytc_w8_n2_nt", 8192, 8192},
    {16, false, true, "skinnytc_w16_n2_nt", 0, 8192},
    {16, false, true, "skinnytl_w16_b1_k64_nt"},
    {8, false, true, "skinnyt_m8_j4_u2_nt"},
    {16, false, true, "skinnytm_w8_j1_u4_nt"},
    {8, true, true, "skinnytc_w8_n2_tt", 8192, 8192},
    {16, true, true, "skinnytc_w16_n2_tt", 0, 8192},
    {16, true, true, "skinnytl_w16_b1_k64_tt"},
    {16, true, true, "skinnytm_w8_j1_u4_tt"},
};

// K split of the "_sk_" MFMA entries: used only when the tile grid has fewer
// than kSplitKBelowWorkgroups workgroups; then K is cut into slices of at
// least kSplitKMinKTiles K-tiles so that tiles x slices reaches about
// kSplitKTargetWorkgroups (four per CU).
constexpr int64_t kSplitKBelowWorkgroups = 512;
constexpr int64_t kSplitKTargetWorkgroups = 1024;
constexpr int64_t kSplitKMinKTiles = 8;

}  // namespace gemmf32
