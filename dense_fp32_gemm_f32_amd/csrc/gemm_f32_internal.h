// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

// The kernel table of the default build holds the kernels the tuning tables
// can pick (and the reference kernel).  Building with -DGEMM_F32_SWEEP=1 adds
// the variants tuning sweeps compare them with: other tiles, schedules and load
// widths, the _nn twins of the transposed-layout kernels, and a K-split
// ("_sk_") twin of every MFMA tile kernel.
#ifndef GEMM_F32_SWEEP
#define GEMM_F32_SWEEP 0
#endif

namespace gemmf32 {

// One GEMM call after validation: C[i*ldc+j] = sum_k A[i*lda+k] * B[k*ldb+j]
// for 0 <= i < M, 0 <= j < N.  M, N, K fit in int32; pitches are 64-bit.
struct Problem {
  const float* A;
  const float* B;
  float* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  // Strided batch: product b (0 <= b < batch, blockIdx.z) reads A + b*sa and
  // B + b*sb and writes C + b*sc.  A single product has batch == 1.  Only the
  // whole-K MFMA kernels, the reference kernel and the K == 0 fill take
  // batch > 1; the others reject it at launch.
  int64_t sa = 0, sb = 0, sc = 0;
  int batch = 1;
};

// The update written to each element of C, given its fp32 sum s and column j:
//   C = act(alpha * s + beta * C + bias[j])
// C is not read when beta == 0; bias may be NULL; act 0 is the identity and 1
// is ReLU, relu(x) = (x < 0 ? +0 : x), which keeps NaN.  The plain product is
// alpha = 1, beta = 0, no bias, identity.
struct Epilogue {
  float alpha = 1.f, beta = 0.f;
  const float* bias = nullptr;
  int act = 0;
};

#if defined(__HIP__)
__device__ __forceinline__ float epilogue_apply(const Epilogue& e, float s, const float* c,
                                                int64_t j) {
  float v = e.alpha * s;
  if (e.beta != 0.f) v = v + e.beta * *c;
  if (e.bias) v = v + e.bias[j];
  if (e.act == 1 && v < 0.f) v = 0.f;
  return v;
}

// Point p at product blockIdx.z of a strided batch.
__device__ __forceinline__ void select_batch(Problem& p) {
  const int64_t b = blockIdx.z;
  p.A += b * p.sa;
  p.B += b * p.sb;
  p.C += b * p.sc;
}
#endif

// Largest batch of one launch (grid z); larger batches are launched in chunks.
constexpr int kMaxLaunchBatch = 65535;

// ---- macro-tiled fp32 MFMA kernel --------------------------------------
// slices == 1: one workgroup per output tile over all of K, writing C.
// slices > 1: K is cut into slices of kchunk (a multiple of bk); slice s
// writes its partial product to partials + s*M*N (pitch N) and a combine
// dispatch sums the slices into C in slice order.
struct MfmaVariant {
  const char* name;
  int bm, bn, bk;      // workgroup tile
  int wm, wn;          // wave tile
  bool vec_a, vec_b;   // 128-bit global loads of A / B (any pitch, 4-byte aligned)
  // Direct global -> LDS loads.  These need A and B 16-byte aligned, lda, ldb
  // and N multiples of 4 and K a multiple of bk.
  bool lds_dma;
  // e: the update written to C (applied by the combine when K is split)
  hipError_t (*launch)(const Problem&, int slices, int kchunk, float* partials, const Epilogue& e,
                       hipStream_t);
  // Direct global -> LDS copies of single floats: any pitch and alignment, K
  // at least two K-tiles, no K split, and 32-bit offsets within a tile
  // (bm lda and bk ldb below 2^29 floats).
  bool copy4 = false;
};
int mfma_variant_count();          // all three kinds below
const MfmaVariant& mfma_variant(int i);
int mfma_dma_variant_count();      // the direct-to-LDS kernels
const MfmaVariant& mfma_dma_variant(int i);
int mfma_small_variant_count();    // fragments from global memory, K split over waves
const MfmaVariant& mfma_small_variant(int i);
int mfma_dma_ks_variant_count();   // direct-to-LDS loads, K-tiles shared by wave groups
const MfmaVariant& mfma_dma_ks_variant(int i);
int mfma_d4_variant_count();       // direct-to-LDS copies of single floats, any pitch
const MfmaVariant& mfma_d4_variant(int i);

// ---- MFMA kernel for C = alpha * op(A) op(B) + beta * C ------------------
// trans_a: A stored K x M (op(A) = A^T); trans_b: B stored N x K.  The
// Problem's lda / ldb are the pitches of the stored matrices.
struct MfmaExVariant {
  const char* name;
  int bm, bn, bk;
  bool trans_a, trans_b;
  hipError_t (*launch)(const Problem&, const Epilogue&, hipStream_t);
  // direct-to-LDS loads: A and B 16-byte aligned, lda and ldb multiples of 4,
  // K a multiple of bk, M (A^T) or N (B as is) a multiple of 4
  bool lds_dma = false;
};
// The register-staged kernels (kernels_mfma_ex.hip), then the direct-to-LDS
// ones (kernels_mfma_ex_dma.hip).
int mfma_ex_variant_count();
const MfmaExVariant& mfma_ex_variant(int i);
int mfma_ex_dma_variant_count();
const MfmaExVariant& mfma_ex_dma_variant(int i);

// ---- skinny-M kernels (M <= 16) --------------------------------------------
// Three kernels: B stored K x N (column tiles x K slices, MFMA; kernels_skinny.hip,
// with the slices added by a second dispatch or in-kernel through exchange slots),
// the same with KiB row runs when B's rows are 16-byte aligned
// (kernels_skinny_rows.hip), and B stored N x K (rows of B^T streamed whole;
// kernels_skinny_t.hip).  Both
// take A as is or transposed (trans_a) and write C = alpha * A B + beta * C,
// directly or through the K-slice partials and the combine.
struct SkinnyPlan {
  int splits;              // K slices (workgroups along K for one column tile)
  int kslice;              // K per slice, in the kernel's units (see its plan)
  int strips;              // workgroups along N
  size_t partial_floats;   // workspace floats for the partial sums (0 if splits == 1)
  size_t lds_bytes;        // dynamic LDS
  // Kernels that add their K slices in-kernel through exchange slots: the
  // 64-bit slots needed (0 for the others), and the slots themselves, which
  // the dispatcher fills in.  The slots are all zero before a launch and the
  // kernel leaves them zero.
  size_t slot_words = 0;
  unsigned long long* slots = nullptr;
};
struct SkinnyVariant {
  const char* name;
  int mr;              // rows of A handled (M <= mr)
  int waves;           // waves per workgroup
  int unroll;          // loads in flight per wave
  bool vec_a;          // 128-bit loads of A (needs 16-byte A rows)
  bool vec_b;          // wide loads of B (needs 16-byte B rows)
  int target_splits;   // K slices (0 = choose from the shape)
  bool trans_a, trans_b;
  SkinnyPlan (*plan)(const Problem&, int target_splits);
  hipError_t (*launch)(const Problem&, const SkinnyPlan&, float* partials, const Epilogue&,
                       hipStream_t);
  // needs B 16-byte aligned with ldb a multiple of 4 (whole 16-byte units of
  // its rows), and N a multiple of 4 too when B is stored K x N
  bool b16 = false;
  // needs A 16-byte aligned with lda a multiple of 4
  bool a16 = false;
};
int skinny_variant_count();          // all three kernels
const SkinnyVariant& skinny_variant(int i);
int skinny_t_variant_count();        // B stored N x K
const SkinnyVariant& skinny_t_variant(int i);
int skinny_rows_variant_count();     // B stored K x N, KiB row runs
const SkinnyVariant& skinny_rows_variant(int i);
int skinny_tm_variant_count();       // B stored N x K, on the matrix cores
const SkinnyVariant& skinny_tm_variant(int i);

// ---- sum of K-slice partials: C = part[0] + part[1] + ... (slice order) ---
// With alpha and beta: C = alpha * (sum of slices) + beta * C (C not read when beta == 0).
hipError_t launch_combine(const Problem& p, int slices, const float* partials, hipStream_t s,
                          const Epilogue& e = Epilogue{});

// ---- deterministic sum of an fp32 array ------------------------------------
// Pass 1: `groups` workgroups, group g sums x[g*chunk, min(n, (g+1)*chunk));
// pass 2, in group 0 of the same dispatch, adds the partials into *out.  Both
// depend on n only.
struct ReducePlan {
  int groups = 0;      // 0 for n == 0 (a one-thread kernel writes +0.0)
  int64_t chunk = 0;   // elements per group, a multiple of 4
};
ReducePlan plan_reduce(int64_t n);
// slots: exchange slots (plan_reduce(n).groups words; may be null for one
// group), all zero before the launch and left zero by it
hipError_t launch_reduce_sum(int64_t n, const float* x, float* out, unsigned long long* slots,
                             hipStream_t s);

// ---- the fixed scratch array of gemm_f32_noalloc (scratch_static.hip) ------
// Device addresses of this device's copy: the exchange slots (all zero
// between calls) and the partial-sum floats.  Looked up, and the slots
// cleared, on the first call per device; GEMM_F32_ERR_WORKSPACE if that first
// call is on a stream being captured, GEMM_F32_ERR_LAUNCH if the clear fails.
struct NoallocScratch {
  unsigned long long* slots = nullptr;
  size_t slot_words = 0;
  float* partials = nullptr;
  size_t partial_floats = 0;
};
int noalloc_scratch(int dev, hipStream_t s, NoallocScratch* out);

// ---- the shader clock under fp32 MFMA load (clock_probe.hip) ---------------
// kClockProbeWorkgroups workgroups of 4 waves, each wave 4 x iters MFMAs;
// workgroup w writes [s_memtime, s_memrealtime] at its start and end to
// stamps[4w .. 4w + 3].
constexpr int kClockProbeWorkgroups = 1024;
hipError_t launch_clock_probe(int iters, unsigned long long* stamps, hipStream_t s);

// ---- naive reference and the K == 0 fill ----------------------------------
hipError_t launch_ref(const Problem& p, hipStream_t s);
// C = beta * C over the M x N window (C = +0.0 when beta == 0; C not read then)
hipError_t launch_scale(const Problem& p, const Epilogue& e, hipStream_t s);

}  // namespace gemmf32
