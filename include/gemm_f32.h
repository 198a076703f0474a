/*
 * gemm_f32.h -- C ABI of the MI355X (gfx950) dense fp32 GEMM library.
 *
 * Operation.  C = A x B for row-major fp32 matrices: A is M x K, B is K x N,
 * C is M x N, and element (i, j) of C is row i of A dotted with column j of B.
 * This is the operation every kernel of "Optimizing a WebGPU Matmul Kernel
 * using Subgroups" computes (section 1 Naive defines it, sections 2-8 keep
 * it), that "WebGPU 行列積の限界を測る" states as C = A x B for N x N
 * matrices, and that the ybb.press page and "WebGPU WGSL Compute Shaders:
 * Custom Matrix Multiplication (GEMM) Optimization Guide" (section 4) write
 * with separate M, N, K sizes and guarded edges.
 *
 * Arithmetic.  Products and sums are fp32 (the pages accumulate in an f32
 * variable).  The order of the K-term summation is not specified; results on
 * small-integer inputs are exact, and on general inputs every element is
 * within the usual fp32 summation error of the exact dot product.
 * Bitwise-identical inputs on the same device give bitwise-identical outputs.
 *
 * Layout.  Row-major with leading dimensions (row pitches, in elements):
 *   A[i*lda + k], B[k*ldb + j], C[i*ldc + j].
 * Required: lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N).
 * Only the M x N window of C is written; the rest of each C row (the pitch
 * padding) and everything outside the window is never read or written.
 * C's previous contents are never read (C is overwritten, no alpha/beta).
 * K == 0 writes +0.0 to the window.  M == 0 or N == 0 is a successful no-op.
 *
 * Memory and ownership.  A, B and C are caller-owned device memory that the
 * current HIP device can access (hipMalloc or a torch CUDA/HIP tensor).  The
 * library keeps no reference to them after the call returns.  It owns only
 * its code objects and, for the kernels that split K over workgroups (the
 * skinny-M kernels and the K-split MFMA entries), scratch workspaces (per
 * device and stream, allocated on first need, freed by
 * gemm_f32_release_workspaces or at unload): per-slice partial sums, or the
 * exchange slots in which the skinny-M kernel adds its K slices.  The slots
 * are cleared once when allocated and every call leaves them clear.  A
 * workspace that a larger call outgrows is replaced but kept, not freed,
 * until gemm_f32_release_workspaces.  C must not overlap A or B.
 *
 * Graph capture.  Every call may be captured into a HIP graph: a call
 * enqueues no host synchronisation, and no memset except the one that clears
 * newly allocated exchange slots.  A call that needs a workspace and would
 * have to allocate or grow it on a stream that is being captured returns
 * GEMM_F32_ERR_WORKSPACE instead: make the same call once on that stream
 * before capturing.  A captured graph keeps the workspace of the stream it
 * was captured on, which stays valid when later calls outgrow it (until
 * gemm_f32_release_workspaces); replays of it must not overlap other work
 * that uses the same workspace (calls on that stream, or other replays).
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Work is enqueued on it and the call returns without waiting; the
 * caller synchronises.  Calls on one stream are ordered by the stream; calls
 * on different streams may run concurrently (each stream has its own
 * workspace).
 *
 * Errors.  Every function returns a status; no exceptions cross the ABI and
 * there is no global error state.  Arguments are checked before anything is
 * enqueued -- dimensions, pitches, NULL pointers, 4-byte alignment of the
 * pointers (the natural alignment of float), aliasing, the device, and last
 * whether the device can reach the pointers -- so a bad call changes nothing.  Sizes above
 * GEMM_F32_MAX_DIM in M, N or K are rejected as GEMM_F32_ERR_INVALID_DIM.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_F32_VERSION 5

/* Activations of gemm_f32_fused. */
#define GEMM_F32_ACT_NONE 0
#define GEMM_F32_ACT_RELU 1   /* relu(x) = (x < 0 ? +0 : x): NaN stays NaN */

/* Largest accepted M, N or K (2^31 - 2^16: tile arithmetic stays in int32). */
#define GEMM_F32_MAX_DIM INT64_C(2147418112)

/* The fixed scratch of gemm_f32_noalloc, per device: exchange slots of the
 * in-kernel K-slice sum, then per-slice partial sums (16 MiB in all). */
#define GEMM_F32_NOALLOC_SLOT_BYTES 4194304
#define GEMM_F32_NOALLOC_PARTIAL_BYTES 12582912

enum gemm_f32_status {
  GEMM_F32_OK = 0,
  GEMM_F32_ERR_INVALID_DIM = 1,   /* M, N or K negative or above GEMM_F32_MAX_DIM */
  GEMM_F32_ERR_INVALID_LD = 2,    /* a pitch below the row length (or below 1) */
  GEMM_F32_ERR_NULL_PTR = 3,      /* NULL A, B or C where the matrix has elements */
  GEMM_F32_ERR_ALIAS = 4,         /* C's extent overlaps A's or B's */
  GEMM_F32_ERR_DEVICE = 5,        /* no HIP device, or the current one is not gfx950 */
  GEMM_F32_ERR_WORKSPACE = 6,     /* scratch workspace could not be allocated */
  GEMM_F32_ERR_LAUNCH = 7,        /* the kernel launch reported an error */
  GEMM_F32_ERR_BAD_KERNEL = 8,    /* unknown kernel index, or one that cannot run these arguments */
  GEMM_F32_ERR_POINTER = 9,       /* A, B or C not 4-byte aligned, or not memory the current device can access */
  GEMM_F32_ERR_INVALID_ARG = 10,  /* an activation other than GEMM_F32_ACT_NONE / _RELU */
  GEMM_F32_ERR_SCRATCH = 11       /* gemm_f32_noalloc: the call needs more scratch than its fixed array */
};

/*
 * gemm_f32 -- C = A x B with the kernel the dispatcher picks from the gfx950
 * tuning table (a macro-tiled MFMA kernel, with K split over workgroups for
 * small grids; the skinny-M kernel for M <= 16; or the K == 0 fill).  The
 * tiled kernels follow "Optimizing a WebGPU Matmul Kernel using Subgroups"
 * (sections 2-8: workgroup tiles, coalesced and 128-bit loads, shared-memory
 * tiles, register blocking, a matrix instruction) and the guarded tiles of
 * the GEMM Optimization Guide (section 4); the K split and its second pass
 * follow "GPU compute shaders" (How it works, step 6).  Arguments as
 * described above.
 *
 * Speed: A and B 16-byte aligned, lda, ldb and N multiples of 4 and K a
 * multiple of 32 (16 for some tiles) let the dispatcher take the kernels that
 * load tiles straight from global memory into LDS; any other 4-byte aligned
 * operands run register-staged kernels of the same tiles, typically 5-25 %
 * slower.
 */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/*
 * gemm_f32_noalloc -- gemm_f32 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, checks, kernel choice and result as gemm_f32,
 * bit for bit; the kernels that split K over workgroups take their scratch
 * from a fixed array compiled into the library instead of a per-stream
 * workspace, so no call allocates or frees anything.
 *
 * The array is GEMM_F32_NOALLOC_SLOT_BYTES of exchange slots plus
 * GEMM_F32_NOALLOC_PARTIAL_BYTES of partial sums, one copy per device, held
 * from the library's load until the process ends.  A call whose kernel needs
 * more than either region returns GEMM_F32_ERR_SCRATCH and enqueues nothing
 * (only M <= 16 products split K: e.g. 8 x 28672 x 4096 needs 7.3 MB of
 * partial sums, 8 x 8192 x 8192 1 MiB of slots; gemm_f32 has no such limit).
 * The first call on each device looks the array up and clears the slot region,
 * waiting for that on `stream`; when that first call is on a stream being
 * captured it returns GEMM_F32_ERR_WORKSPACE instead (make one call outside
 * capture first).  Every call on a device shares that device's array: calls
 * that may overlap on one device (other streams, graph replays) race and must
 * be ordered by the caller.  gemm_f32, gemm_f32_ex and the others keep their
 * own workspaces and never touch the array.
 */
int gemm_f32_noalloc(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     void *stream);

/*
 * gemm_f32_ex -- C = alpha * op(A) op(B) + beta * C, the BLAS-style form for
 * row-major storage.  op(A) is A (stored M x K, element (i, k) at A[i*lda + k])
 * when transA == 0, and A^T (A stored K x M, element (i, k) at A[k*lda + i])
 * otherwise; op(B) is B (stored K x N) when transB == 0 and B^T (B stored
 * N x K, element (k, j) at B[j*ldb + k]) otherwise.  lda and ldb are the
 * pitches of the stored matrices: lda >= max(1, transA ? M : K), ldb >=
 * max(1, transB ? K : N).  When beta == 0 the input C is not read (so NaN or
 * Inf there does not propagate); otherwise it is read once per element.
 * K == 0 gives C = beta * C.  alpha multiplies the product of the inputs.
 *
 * The pages define only C = A x B; the transposed operands follow the
 * pre-transposed B of "Optimizing a WebGPU Matmul Kernel using Subgroups"
 * (section 7) and the BLAS convention, alpha and beta a fused epilogue (one
 * memory pass fewer, "GPU compute shaders", Performance section).  With A and
 * B as stored it runs the kernels gemm_f32 picks for the shape, which apply
 * alpha and beta as they store C (exactly gemm_f32 when alpha = 1, beta = 0);
 * a transposed operand runs the extended-operation kernels.  Same checks and
 * errors as gemm_f32, with the pitches checked against the stored shapes.
 * Those load tiles straight into LDS under gemm_f32's conditions, with M a
 * multiple of 4 when A is transposed and N a multiple of 4 when B is not.
 */
int gemm_f32_ex(int transA, int transB,
                int64_t M, int64_t N, int64_t K,
                float alpha,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float beta,
                float *C, int64_t ldc,
                void *stream);

/*
 * gemm_f32_fused -- C = act(alpha * op(A) op(B) + beta * C + bias) in one
 * pass: gemm_f32_ex with a bias row vector and an activation applied in the
 * kernel's epilogue, so the product never makes a second trip through HBM
 * ("GPU compute shaders", Performance: fuse kernels, one memory pass fewer).
 * bias: N floats, device memory, bias[j] added to every row's column j (NULL
 * for none; 4-byte aligned, not inside C's window, else GEMM_F32_ERR_POINTER /
 * GEMM_F32_ERR_ALIAS).  activation: GEMM_F32_ACT_NONE or GEMM_F32_ACT_RELU
 * (else GEMM_F32_ERR_INVALID_ARG), applied last.  The fp32 update per element
 * is v = alpha * s; v += beta * C (only when beta != 0); v += bias[j]; then
 * act(v).  K == 0 gives act(alpha * 0 + beta * C + bias).  A and B as stored
 * run the kernels gemm_f32 picks (the epilogue is part of every tile
 * kernel's store, and of the combine when K is split); a transposed operand
 * runs the extended-operation kernels.  With no bias and no activation it is
 * exactly gemm_f32_ex.  Other arguments, checks and errors as gemm_f32_ex.
 */
int gemm_f32_fused(int transA, int transB,
                   int64_t M, int64_t N, int64_t K,
                   float alpha,
                   const float *A, int64_t lda,
                   const float *B, int64_t ldb,
                   float beta,
                   float *C, int64_t ldc,
                   const float *bias, int activation,
                   void *stream);

/*
 * gemm_f32_batched -- `batch` independent products C_b = A_b x B_b, 0 <= b <
 * batch, in as few launches as possible: A_b = A + b * strideA, B_b = B + b *
 * strideB, C_b = C + b * strideC (strides in elements), each matrix as for
 * gemm_f32 (row-major with pitches lda, ldb, ldc).  strideA or strideB may be
 * 0 (one matrix shared by every product); the C windows of the products must
 * not overlap (strideC >= (M - 1) * ldc + N, else GEMM_F32_ERR_ALIAS) and no C
 * may overlap any A or B of the batch (GEMM_F32_ERR_ALIAS).  Negative strides
 * give GEMM_F32_ERR_INVALID_LD, a negative batch GEMM_F32_ERR_INVALID_DIM;
 * batch == 0 is a successful no-op and batch == 1 is exactly gemm_f32.
 *
 * The pages time one product per dispatch and find the per-dispatch cost
 * dominant for small sizes, gone when dispatches are batched ("GPU compute
 * shaders", Performance); this is that batching for a run of small products:
 * one launch covers every tile of every product (grid z = product), with the
 * whole-K MFMA kernels chosen by the same table from the batch's total tile
 * count.  Each product is summed as gemm_f32 sums a product of its class:
 * exact on small integers, within fp32 summation error otherwise.  Other
 * checks, errors, ownership and stream behaviour as gemm_f32.
 */
int gemm_f32_batched(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, int64_t strideA,
                     const float *B, int64_t ldb, int64_t strideB,
                     float *C, int64_t ldc, int64_t strideC,
                     int64_t batch, void *stream);

/*
 * gemm_f32_ref_gpu -- the same operation with the naive one-thread-per-output
 * kernel ("Optimizing a WebGPU Matmul Kernel using Subgroups", sections 1-3:
 * one invocation per element of C, adjacent threads on adjacent columns, k
 * ascending with fp32 fused multiply-add).  Slow; for debugging and as a
 * second GPU witness.  Same arguments, checks and errors as gemm_f32.
 */
int gemm_f32_ref_gpu(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     void *stream);

/*
 * reduce_sum_f32 -- *out = x[0] + x[1] + ... + x[n-1] for n fp32 values in
 * device memory, summed in fp32 in an order that depends on n only, so the
 * same array gives bitwise the same result on every run and at any address.
 *
 * The reduction of "GPU compute shaders" (How it works: one partial sum per
 * workgroup from a grid-stride loop and a shared-memory tree, then the
 * partials combined; the Pitfalls section's fixed group count and order for
 * a reproducible result), measured there on 2^26 values.  One launch: up to
 * 256 workgroups each sum a contiguous chunk; each hands its partial to
 * workgroup 0 through a per-stream exchange slot (a flag and the value in one
 * 64-bit word, written with a device-scope atomic), and workgroup 0 adds the
 * partials in index order and writes *out.  Workgroup 0 waits only on
 * workgroups that never wait, so the launch always completes; should a
 * partial still be missing after about 2^20 polls of its slot (seconds, so
 * only a GPU held by other work that long could cause it), *out is NaN and
 * the late partial may be left in its slot: then call
 * gemm_f32_release_workspaces before the next call on that stream, which
 * would otherwise read it.  The error is at most about
 * d 2^-24 sum|x[i]|, with d the depth of the summation tree (276 for n =
 * 2^26; d grows as n / 2^18 beyond that); exact when every partial sum is
 * an integer below 2^24 in magnitude.  n == 0 writes +0.0.  NaN and Inf
 * propagate as IEEE addition does.
 *
 * x: n floats (4-byte aligned; 16-byte aligned reads at full width); out: one
 * float, not inside x.  Both device memory of the current device, caller
 * owned.  Errors: n < 0 GEMM_F32_ERR_INVALID_DIM; NULL x (n > 0) or out
 * GEMM_F32_ERR_NULL_PTR; misaligned or unreachable pointers
 * GEMM_F32_ERR_POINTER; out inside x GEMM_F32_ERR_ALIAS; then the device and
 * workspace checks of gemm_f32 (it uses the per-stream exchange slots of the
 * skinny kernels, which every call leaves clear).
 * Asynchronous on `stream` like gemm_f32.
 */
int reduce_sum_f32(int64_t n, const float *x, float *out, void *stream);

/*
 * gemm_f32_clock_probe -- for measurement records: the shader clock the GPU
 * sustains under fp32 matrix-core load at the time of the call.  The fp32
 * MFMA peak is 256 FLOP per clock per CU, so a throughput is read against
 * the clock it ran at ("GPU compute shaders", Performance: GPU-timed runs).
 * Launches GEMM_F32_CLOCK_PROBE_WORKGROUPS workgroups of 4 waves (4 per CU on
 * MI355X, every SIMD busy), each wave issuing 4 * iters
 * v_mfma_f32_32x32x2_f32 on registers only (about 1 ms for iters = 2400).
 * Workgroup w writes four 64-bit words to stamps[4w .. 4w + 3]: the shader
 * cycle counter (s_memtime) and the constant-rate counter (s_memrealtime)
 * after a barrier at its start, then both again after a barrier at its end.
 * The achieved clock in kHz is wall_khz * (word 2 - word 0) / (word 3 - word
 * 1).  stamps: device memory of 4 * GEMM_F32_CLOCK_PROBE_WORKGROUPS uint64,
 * caller-owned.  wall_khz, max_khz: host ints (either may be NULL) that
 * receive the constant counter's rate (hipDeviceAttributeWallClockRate) and
 * the device's peak shader clock (hipDeviceAttributeClockRate), in kHz.
 * Errors: iters outside [1, 2^24] GEMM_F32_ERR_INVALID_DIM; NULL stamps
 * GEMM_F32_ERR_NULL_PTR; stamps not 8-byte aligned or not reachable
 * GEMM_F32_ERR_POINTER; then the device check of gemm_f32.  The kernel is
 * asynchronous on `stream`; the two rates are written before the call returns.
 */
#define GEMM_F32_CLOCK_PROBE_WORKGROUPS 1024
int gemm_f32_clock_probe(int64_t iters, unsigned long long *stamps, int *wall_khz,
                         int *max_khz, void *stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *gemm_f32_status_string(int status);

/*
 * gemm_f32_selected_kernel -- name of the tuning-table entry gemm_f32 would
 * run for these arguments ("empty", "fill_zero_k0", or a kernel name).  Pure
 * host logic: touches no device and enqueues nothing.  The pointers are only
 * inspected for alignment.  Returns "invalid" for arguments gemm_f32 would
 * reject on dimensions or pitches.
 */
const char *gemm_f32_selected_kernel(int64_t M, int64_t N, int64_t K,
                                     int64_t lda, int64_t ldb, int64_t ldc,
                                     const void *A, const void *B, const void *C);

/* gemm_f32_selected_kernel for gemm_f32_ex's arguments. */
const char *gemm_f32_selected_kernel_ex(int transA, int transB,
                                        int64_t M, int64_t N, int64_t K,
                                        int64_t lda, int64_t ldb, int64_t ldc,
                                        float alpha, float beta,
                                        const void *A, const void *B, const void *C);

/* gemm_f32_selected_kernel for gemm_f32_batched's arguments (strides of A
 * and B; the kernel is the same whatever C's stride). */
const char *gemm_f32_selected_kernel_batched(int64_t M, int64_t N, int64_t K,
                                             int64_t lda, int64_t strideA,
                                             int64_t ldb, int64_t strideB, int64_t ldc,
                                             int64_t batch, const void *A, const void *B);

/* Library version (GEMM_F32_VERSION). */
int gemm_f32_version(void);

/*
 * Kernel table access, for tuning sweeps and for tests that exercise every
 * kernel variant.  Index range [0, gemm_f32_kernel_count()).
 * gemm_f32_kernel_name returns NULL for an index out of range.
 * gemm_f32_run_kernel runs entry `index` exactly as gemm_f32 would run it if
 * the dispatcher had picked it; entries that cannot handle the arguments
 * (a direct-to-LDS variant, named "..._d6_...", without 16-byte aligned A and
 * B, lda, ldb and N multiples of 4 and K a multiple of its K-tile; or a
 * skinny variant with more than 16 rows) return GEMM_F32_ERR_BAD_KERNEL and
 * enqueue nothing.
 */
int gemm_f32_kernel_count(void);
const char *gemm_f32_kernel_name(int index);
int gemm_f32_run_kernel(int index,
                        int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda,
                        const float *B, int64_t ldb,
                        float *C, int64_t ldc,
                        void *stream);

/*
 * gemm_f32_run_kernel_ex -- gemm_f32_run_kernel with gemm_f32_ex's arguments.
 * The "mfmaex_..._<ab>" entries take the layout ab (n: stored as is, t:
 * stored transposed) with any alpha and beta; every other entry takes only
 * transA = transB = 0, alpha = 1, beta = 0.  Otherwise GEMM_F32_ERR_BAD_KERNEL.
 */
int gemm_f32_run_kernel_ex(int index, int transA, int transB,
                           int64_t M, int64_t N, int64_t K,
                           float alpha,
                           const float *A, int64_t lda,
                           const float *B, int64_t ldb,
                           float beta,
                           float *C, int64_t ldc,
                           void *stream);

/*
 * gemm_f32_run_kernel_fused -- gemm_f32_run_kernel_ex with gemm_f32_fused's
 * bias and activation (the same kernels take them).
 */
int gemm_f32_run_kernel_fused(int index, int transA, int transB,
                              int64_t M, int64_t N, int64_t K,
                              float alpha,
                              const float *A, int64_t lda,
                              const float *B, int64_t ldb,
                              float beta,
                              float *C, int64_t ldc,
                              const float *bias, int activation,
                              void *stream);

/*
 * gemm_f32_release_workspaces -- free every scratch workspace the library
 * holds (all devices, all streams, outgrown ones included) after
 * synchronising the devices they live on.  Safe to call at any time no call
 * is in flight from another thread; graphs captured before it must not be
 * replayed after it.
 */
int gemm_f32_release_workspaces(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
