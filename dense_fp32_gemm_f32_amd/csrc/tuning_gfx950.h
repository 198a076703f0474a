// Tuning table for gfx950 (MI355X): which kernel gemm_f32 runs for a shape.
//
// The first row whose bounds hold wins.  A row names a kernel family; the
// dispatcher appends the load-width suffix the operands allow ("_vec" when
// the rows of A and B are 16-byte aligned, otherwise "_veca", "_vecb" or
// "_scalar"; skinny rows: "_vec" or "_scalar" for B).
//
// Columns:
//   max_m       the row applies when M <= max_m
//   min_tiles   ... and the grid of 128 x 128 tiles has at least this many tiles
//   kernel      kernel family (a name prefix in the kernel table)
#pragma once

#include <cstdint>

namespace gemmf32 {

struct TuningRow {
  int64_t max_m;
  int64_t min_tiles;
  const char* kernel;
};

constexpr int64_t kAnyM = INT64_C(0x7fffffff);

constexpr TuningRow kTuningGfx950[] = {
    {4, 0, "skinny_m4_w4_u8_s0"},
    {8, 0, "skinny_m8_w4_u8_s0"},
    {16, 0, "skinny_m16_w4_u4_s0"},
    {kAnyM, 256, "mfma_128x128x16_w64x64"},
    {kAnyM, 0, "mfma_64x64x16_w32x32"},
};

}  // namespace gemmf32
