// C ABI of the gfx950 fp32 GEMM library: argument checks, the tuning-table
// dispatcher, the workspace for K-slice partial sums, and the kernel table.
//
// The pages pass caller-created buffers and M, N, K to one GEMM entry point
// ("WebGPU WGSL Compute Shaders: Custom Matrix Multiplication (GEMM)
// Optimization Guide", section 5, and the dimensions uniform of the ybb.press
// page); this library takes device pointers, sizes, row pitches and a HIP
// stream instead, and reports errors with status codes.
#include "../../include/gemm_f32.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "gemm_f32_internal.h"
#include "read_probe.h"
#include "stamps.h"
#include "tuning_gfx950.h"
#if GEMM_F32_SWEEP
#include "../../include/gemm_f32_sweep.h"
#endif

using gemmf32::Problem;

namespace {

// ---- kernel table: MFMA variants (whole K; with GEMM_F32_SWEEP also K
// split), extended-operation and skinny variants, the naive kernel ----------
enum class Kind { Mfma, MfmaSplitK, MfmaEx, Skinny, Ref };
struct Entry {
  Kind kind;
  int sub;           // index within its family
  std::string name;  // never changes once the table is built
};

// "mfma_<tile>_<width>" -> "mfma_<tile>_sk_<width>"
std::string split_k_name(const std::string& name) {
  const size_t cut = name.rfind('_');
  return name.substr(0, cut) + "_sk" + name.substr(cut);
}

const std::vector<Entry>& entries() {
  static const std::vector<Entry> table = [] {
    std::vector<Entry> t;
    for (int i = 0; i < gemmf32::mfma_variant_count(); ++i)
      t.push_back({Kind::Mfma, i, gemmf32::mfma_variant(i).name});
#if GEMM_F32_SWEEP
    // K-split twins: the tuning table picks none of them (none for the
    // single-float copy tiles, which take no K split)
    for (int i = 0; i < gemmf32::mfma_variant_count(); ++i)
      if (!gemmf32::mfma_variant(i).copy4)
        t.push_back({Kind::MfmaSplitK, i, split_k_name(gemmf32::mfma_variant(i).name)});
#endif
    for (int i = 0; i < gemmf32::mfma_ex_variant_count(); ++i)
      t.push_back({Kind::MfmaEx, i, gemmf32::mfma_ex_variant(i).name});
    for (int i = 0; i < gemmf32::skinny_variant_count(); ++i)
      t.push_back({Kind::Skinny, i, gemmf32::skinny_variant(i).name});
    t.push_back({Kind::Ref, 0, "ref_naive"});
    return t;
  }();
  return table;
}

int find_entry(const std::string& name) {
  const auto& t = entries();
  for (size_t i = 0; i < t.size(); ++i)
    if (name == t[i].name) return (int)i;
  return -1;
}

// K split of an MFMA entry: slices of whole K-tiles, enough workgroups to
// fill the GPU when the tile grid alone does not (see tuning_gfx950.h).
struct MfmaPlan {
  int slices;
  int kchunk;
};
MfmaPlan plan_mfma(const gemmf32::MfmaVariant& v, const Problem& p, bool split) {
  const MfmaPlan whole{1, p.K};
  if (!split) return whole;
  const int64_t tiles = (int64_t)((p.M + v.bm - 1) / v.bm) * ((p.N + v.bn - 1) / v.bn);
  const int64_t ktiles = (p.K + v.bk - 1) / v.bk;
  if (tiles >= gemmf32::kSplitKBelowWorkgroups) return whole;
  int64_t slices = (gemmf32::kSplitKTargetWorkgroups + tiles - 1) / tiles;
  const int64_t cap = ktiles / gemmf32::kSplitKMinKTiles;
  if (slices > cap) slices = cap;
  if (slices <= 1) return whole;
  const int64_t per = (ktiles + slices - 1) / slices;   // K-tiles per slice
  slices = (ktiles + per - 1) / per;                     // no empty slice
  if (slices <= 1) return whole;
  return MfmaPlan{(int)slices, (int)(per * v.bk)};
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The operation around the product: C = act(alpha * op(A) op(B) + beta * C +
// bias), with op(A) = A^T when ta (A stored K x M) and op(B) = B^T when tb (B
// stored N x K); bias a row of N values or NULL; act 0 identity, 1 ReLU.
struct Op {
  bool ta = false, tb = false;
  float alpha = 1.f, beta = 0.f;
  const float* bias = nullptr;
  int act = 0;
  bool plain() const {
    return !ta && !tb && alpha == 1.f && beta == 0.f && !bias && act == 0;
  }
  gemmf32::Epilogue epilogue() const {
    gemmf32::Epilogue e;
    e.alpha = alpha;
    e.beta = beta;
    e.bias = bias;
    e.act = act;
    return e;
  }
};

// ---- argument checks (host only, nothing enqueued) -------------------------
int check_args(const Op& op, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
               const float* B, int64_t ldb, const float* C, int64_t ldc) {
  const int64_t kMax = GEMM_F32_MAX_DIM;
  if (M < 0 || N < 0 || K < 0 || M > kMax || N > kMax || K > kMax)
    return GEMM_F32_ERR_INVALID_DIM;
  // stored shapes: A is a_rows x a_cols, B is b_rows x b_cols
  const int64_t a_rows = op.ta ? K : M, a_cols = op.ta ? M : K;
  const int64_t b_rows = op.tb ? N : K, b_cols = op.tb ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return GEMM_F32_ERR_INVALID_LD;
  // byte extents must stay far from overflow
  const int64_t kMaxElems = INT64_C(1) << 60;
  if ((a_rows > 0 && lda > kMaxElems / a_rows) || (b_rows > 0 && ldb > kMaxElems / b_rows) ||
      (M > 0 && ldc > kMaxElems / M))
    return GEMM_F32_ERR_INVALID_LD;
  const bool has_a = M > 0 && K > 0, has_b = K > 0 && N > 0, has_c = M > 0 && N > 0;
  if ((has_a && !A) || (has_b && !B) || (has_c && !C)) return GEMM_F32_ERR_NULL_PTR;
  if ((has_a && !aligned4(A)) || (has_b && !aligned4(B)) || (has_c && !aligned4(C)))
    return GEMM_F32_ERR_POINTER;
  if (has_c) {
    const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)(((M - 1) * ldc + N) * 4);
    if (has_a) {
      const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)(((a_rows - 1) * lda + a_cols) * 4);
      if (c0 < a1 && a0 < c1) return GEMM_F32_ERR_ALIAS;
    }
    if (has_b) {
      const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(((b_rows - 1) * ldb + b_cols) * 4);
      if (c0 < b1 && b0 < c1) return GEMM_F32_ERR_ALIAS;
    }
  }
  // the epilogue: a known activation; a bias row that is aligned and not in C
  if (op.act != 0 && op.act != 1) return GEMM_F32_ERR_INVALID_ARG;
  if (op.bias && has_c) {
    if (!aligned4(op.bias)) return GEMM_F32_ERR_POINTER;
    const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)(((M - 1) * ldc + N) * 4);
    const uintptr_t b0 = (uintptr_t)op.bias, b1 = b0 + (uintptr_t)(N * 4);
    if (c0 < b1 && b0 < c1) return GEMM_F32_ERR_ALIAS;
  }
  return GEMM_F32_OK;
}

// ---- device check: gfx950 only, cached per device ---------------------------
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_DEVICE;
  }
  *dev_out = dev;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_F32_ERR_DEVICE;
      }
      g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    if (g_dev_state[dev] != 1) return GEMM_F32_ERR_DEVICE;
  }
  return GEMM_F32_OK;
}

// A, B and C must be memory the current device can reach.
int check_pointer(const void* p, int dev) {
  if (!p) return GEMM_F32_OK;  // only reached for empty matrices
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_POINTER;
  }
  switch (attr.type) {
    case hipMemoryTypeDevice:
      return attr.device == dev ? GEMM_F32_OK : GEMM_F32_ERR_POINTER;
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      return GEMM_F32_OK;
    case hipMemoryTypeHost:
      return attr.devicePointer ? GEMM_F32_OK : GEMM_F32_ERR_POINTER;
    default:
      return GEMM_F32_ERR_POINTER;
  }
}

// ---- scratch workspaces, one set per (device, stream) -----------------------
// Per-slice partial sums of the combine-based skinny kernels and the split-K
// MFMA entries, and the exchange slots of the in-kernel slice sum.  Kept for
// the life of the process (or until gemm_f32_release_workspaces) and grown on
// demand.  A buffer that is outgrown is retired, not freed: work already
// enqueued, and any graph captured earlier on that stream, may still use it.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
};
std::mutex g_ws_mu;
std::map<std::pair<int, uintptr_t>, Workspace>* g_ws = nullptr;   // partial sums
std::map<std::pair<int, uintptr_t>, Workspace>* g_xs = nullptr;   // exchange slots

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A buffer of at least `need` bytes from `table` for (dev, s).  clear: a new
// buffer is zeroed on the stream before any later work on it (the exchange
// slots start empty).  Caller holds g_ws_mu.
int grow_workspace(std::map<std::pair<int, uintptr_t>, Workspace>*& table, int dev,
                   hipStream_t s, size_t need, bool clear, void** out) {
  if (std::getenv("GEMM_F32_TEST_FAIL_WORKSPACE")) return GEMM_F32_ERR_WORKSPACE;
  if (!table) table = new std::map<std::pair<int, uintptr_t>, Workspace>();
  Workspace& w = (*table)[{dev, (uintptr_t)s}];
  if (w.bytes < need) {
    // a stream being captured into a graph can neither allocate nor clear:
    // the workspace must have been grown by an earlier call on that stream
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_F32_ERR_WORKSPACE;
    }
    if (cap != hipStreamCaptureStatusNone) return GEMM_F32_ERR_WORKSPACE;
    // grow with headroom so alternating shapes do not reallocate
    const size_t bytes = round_up(need + need / 2, 1 << 20);
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_F32_ERR_WORKSPACE;
    }
    if (clear && hipMemsetAsync(p, 0, bytes, s) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return GEMM_F32_ERR_WORKSPACE;
    }
    if (w.ptr) w.retired.push_back(w.ptr);
    w.ptr = p;
    w.bytes = bytes;
  }
  *out = w.ptr;
  return GEMM_F32_OK;
}

int get_workspace(int dev, hipStream_t s, size_t partial_floats, float** partials) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  void* p = nullptr;
  const int rc = grow_workspace(g_ws, dev, s, partial_floats * 4, false, &p);
  *partials = static_cast<float*>(p);
  return rc;
}

// The exchange slots: every kernel that uses them finds them all zero and
// leaves them zero, so a new buffer is cleared once, on the stream, before
// its first use.
int get_exchange_slots(int dev, hipStream_t s, size_t words, unsigned long long** slots) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  void* p = nullptr;
  const int rc = grow_workspace(g_xs, dev, s, words * 8, true, &p);
  *slots = static_cast<unsigned long long*>(p);
  return rc;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("GEMM_F32_LOG");
    return v && *v && *v != '0';
  }();
  return on;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Can entry e run these arguments?  (128-bit loads through registers need only
// the 4-byte alignment checked up front; direct-to-LDS loads need more.)
bool accepts(const Entry& e, const Op& op, int64_t M, int64_t N, int64_t K, int64_t lda,
             int64_t ldb, const void* A, const void* B) {
  if (e.kind == Kind::MfmaEx) {
    const auto& v = gemmf32::mfma_ex_variant(e.sub);
    if (v.trans_a != op.ta || v.trans_b != op.tb) return false;
    if (!v.lds_dma) return true;
    return K >= v.bk && K % v.bk == 0 && lda % 4 == 0 && ldb % 4 == 0 &&
           (!op.ta || M % 4 == 0) && (op.tb || N % 4 == 0) && aligned16(A) && aligned16(B);
  }
  if (e.kind == Kind::Skinny) {
    // any alpha and beta; the layout the kernel was built for
    const auto& v = gemmf32::skinny_variant(e.sub);
    if (M > v.mr || v.trans_a != op.ta || v.trans_b != op.tb) return false;
    if (v.a16 && (lda % 4 != 0 || !aligned16(A))) return false;
    if (v.b16) {
      // whole 16-byte units of B's rows (and, for B stored K x N, of its columns)
      if ((!v.trans_b && N % 4 != 0) || ldb % 4 != 0 || !aligned16(B)) return false;
      Problem p{static_cast<const float*>(A), static_cast<const float*>(B), nullptr, lda, ldb,
                0, (int)M, (int)N, (int)K};
      if (v.plan(p, v.target_splits).splits > 65535) return false;
    }
    return true;
  }
  if (e.kind == Kind::Mfma || e.kind == Kind::MfmaSplitK) {
    // A and B as stored; any epilogue
    if (op.ta || op.tb) return false;
    const auto& v = gemmf32::mfma_variant(e.sub);
    if (v.copy4)
      return e.kind == Kind::Mfma && K >= 2 * v.bk && (int64_t)v.bm * lda < (INT64_C(1) << 29) &&
             (int64_t)v.bk * ldb < (INT64_C(1) << 29);
    if (!v.lds_dma) return true;
    return K % v.bk == 0 && lda % 4 == 0 && ldb % 4 == 0 && N % 4 == 0 && aligned16(A) &&
           aligned16(B);
  }
  // the reference kernel computes the plain product only
  return op.plain();
}
bool entry_accepts(const Entry& e, const Op& op, const Problem& p) {
  return accepts(e, op, p.M, p.N, p.K, p.lda, p.ldb, p.A, p.B);
}

// fixed: the scratch of gemm_f32_noalloc (NULL: this stream's workspaces)
int run_entry(const Entry& e, const Op& op, const Problem& p, int dev, hipStream_t s,
              const gemmf32::NoallocScratch* fixed = nullptr) {
  if (log_enabled())
    std::fprintf(stderr, "[gemm_f32] M=%d N=%d K=%d lda=%lld ldb=%lld ldc=%lld -> %s\n", p.M,
                 p.N, p.K, (long long)p.lda, (long long)p.ldb, (long long)p.ldc,
                 e.name.c_str());
  hipError_t err = hipSuccess;
  switch (e.kind) {
    case Kind::Mfma:
    case Kind::MfmaSplitK: {
      const auto& v = gemmf32::mfma_variant(e.sub);
      const MfmaPlan pl = plan_mfma(v, p, e.kind == Kind::MfmaSplitK);
      float* partials = nullptr;
      if (pl.slices > 1) {
        const size_t need = (size_t)pl.slices * p.M * p.N;
        if (fixed) {
          if (need > fixed->partial_floats) return GEMM_F32_ERR_SCRATCH;
          partials = fixed->partials;
        } else {
          const int rc = get_workspace(dev, s, need, &partials);
          if (rc != GEMM_F32_OK) return rc;
        }
      }
      err = v.launch(p, pl.slices, pl.kchunk, partials, op.epilogue(), s);
      break;
    }
    case Kind::Skinny: {
      const auto& v = gemmf32::skinny_variant(e.sub);
      gemmf32::SkinnyPlan pl = v.plan(p, v.target_splits);
      float* partials = nullptr;
      if (fixed) {
        if (pl.partial_floats > fixed->partial_floats || pl.slot_words > fixed->slot_words)
          return GEMM_F32_ERR_SCRATCH;
        if (pl.partial_floats > 0) partials = fixed->partials;
        if (pl.slot_words > 0) pl.slots = fixed->slots;
      } else {
        if (pl.partial_floats > 0) {
          const int rc = get_workspace(dev, s, pl.partial_floats, &partials);
          if (rc != GEMM_F32_OK) return rc;
        }
        if (pl.slot_words > 0) {
          const int rc = get_exchange_slots(dev, s, pl.slot_words, &pl.slots);
          if (rc != GEMM_F32_OK) return rc;
        }
      }
      err = v.launch(p, pl, partials, op.epilogue(), s);
      break;
    }
    case Kind::MfmaEx:
      err = gemmf32::mfma_ex_variant(e.sub).launch(p, op.epilogue(), s);
      break;
    case Kind::Ref:
      err = gemmf32::launch_ref(p, s);
      break;
  }
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

// ---- the dispatcher ---------------------------------------------------------
// Do the workgroups of an MFMA entry (over `batch` products), `slots` of them
// resident per CU, leave the last wave at least 90 % full, or make four waves
// or more?  (w waves of work take ceil(w) waves of time.)
bool fills_waves(const Entry& e, int64_t M, int64_t N, int64_t batch, int slots) {
  int64_t bm, bn;
  if (e.kind == Kind::Mfma || e.kind == Kind::MfmaSplitK) {
    bm = gemmf32::mfma_variant(e.sub).bm;
    bn = gemmf32::mfma_variant(e.sub).bn;
  } else if (e.kind == Kind::MfmaEx) {
    bm = gemmf32::mfma_ex_variant(e.sub).bm;
    bn = gemmf32::mfma_ex_variant(e.sub).bn;
  } else {
    return true;
  }
  const int64_t wgs = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * batch;
  const int64_t per_wave = gemmf32::kNumCus * slots;
  const int64_t waves = (wgs + per_wave - 1) / per_wave;
  return waves >= 4 || 10 * wgs >= 9 * waves * per_wave;
}

std::string select_name(const Op& op, int64_t M, int64_t N, int64_t K, int64_t lda,
                        int64_t ldb, const void* A, const void* B) {
  if (M == 0 || N == 0) return "empty";
  if (K == 0) return "fill_zero_k0";
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (!op.plain()) {
    for (const auto& row : gemmf32::kTuningGfx950Skinny) {
      if (M > row.max_m || row.ta != op.ta || row.tb != op.tb) continue;
      if (row.max_n > 0 && N > row.max_n) continue;
      if (row.min_k > 0 && K < row.min_k) continue;
      const int idx = find_entry(row.kernel);
      if (idx >= 0 && accepts(entries()[idx], op, M, N, K, lda, ldb, A, B)) return row.kernel;
    }
    // a transposed operand: the extended-operation tiles; A and B as stored
    // (an epilogue only): the plain table below, whose kernels take it
    static const char* const kLayout[2][2] = {{"_nn", "_nt"}, {"_tn", "_tt"}};
    if (op.ta || op.tb) {
      for (const auto& row : gemmf32::kTuningGfx950Ex) {
        if (tiles < row.min_tiles) continue;
        // a row whose kernel cannot take these arguments defers to the next one
        const std::string name = std::string(row.kernel) + kLayout[op.ta][op.tb];
        const int idx = find_entry(name.c_str());
        if (idx < 0 || !accepts(entries()[idx], op, M, N, K, lda, ldb, A, B)) continue;
        if (row.wave_slots > 0 && !fills_waves(entries()[idx], M, N, 1, row.wave_slots)) continue;
        return name;
      }
    }
  }
  for (const auto& row : gemmf32::kTuningGfx950) {
    if (M > row.max_m || tiles < row.min_tiles) continue;
    if (row.max_tiles > 0 && tiles > row.max_tiles) continue;
    // a row whose kernel cannot take these arguments defers to the next one
    const int idx = find_entry(row.kernel);
    if (idx < 0 || !accepts(entries()[idx], op, M, N, K, lda, ldb, A, B)) continue;
    if (row.wave_slots > 0 && !fills_waves(entries()[idx], M, N, 1, row.wave_slots)) continue;
    return row.kernel;
  }
  return "ref_naive";
}

struct Prepared {
  int status;
  int dev;
  Problem p;
};

Prepared prepare(const Op& op, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                 const float* B, int64_t ldb, float* C, int64_t ldc) {
  Prepared r{};
  r.status = check_args(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK) return r;
  r.p = Problem{A, B, C, lda, ldb, ldc, (int)M, (int)N, (int)K};
  if (M == 0 || N == 0) return r;
  r.status = check_device(&r.dev);
  if (r.status != GEMM_F32_OK) return r;
  if (K > 0) {
    if ((r.status = check_pointer(A, r.dev)) != GEMM_F32_OK) return r;
    if ((r.status = check_pointer(B, r.dev)) != GEMM_F32_OK) return r;
  }
  r.status = check_pointer(C, r.dev);
  if (r.status == GEMM_F32_OK && op.bias) r.status = check_pointer(op.bias, r.dev);
  return r;
}

// K == 0: the epilogue of an empty sum, C = act(alpha * 0 + beta * C + bias)
// (+0.0 for the plain product).
int run_k0(const Op& op, const Problem& p, hipStream_t s) {
  if (gemmf32::launch_scale(p, op.epilogue(), s) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

int gemm_impl(const Op& op, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
              const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  Prepared r = prepare(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK || M == 0 || N == 0) return r.status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return run_k0(op, r.p, s);
  const int idx = find_entry(select_name(op, M, N, K, lda, ldb, A, B));
  if (idx < 0) return GEMM_F32_ERR_BAD_KERNEL;
  return run_entry(entries()[idx], op, r.p, r.dev, s);
}

// gemm_f32 with the fixed scratch array instead of the stream's workspaces.
int gemm_noalloc_impl(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  const Op op;
  Prepared r = prepare(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK || M == 0 || N == 0) return r.status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return run_k0(op, r.p, s);
  const int idx = find_entry(select_name(op, M, N, K, lda, ldb, A, B));
  if (idx < 0) return GEMM_F32_ERR_BAD_KERNEL;
  gemmf32::NoallocScratch fixed;
  const int rc = gemmf32::noalloc_scratch(r.dev, s, &fixed);
  if (rc != GEMM_F32_OK) return rc;
  return run_entry(entries()[idx], op, r.p, r.dev, s, &fixed);
}

int run_kernel_impl(int index, const Op& op, int64_t M, int64_t N, int64_t K, const float* A,
                    int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                    void* stream) {
  const auto& t = entries();
  if (index < 0 || index >= (int)t.size()) return GEMM_F32_ERR_BAD_KERNEL;
  Prepared r = prepare(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK || M == 0 || N == 0) return r.status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return run_k0(op, r.p, s);
  if (!entry_accepts(t[index], op, r.p)) return GEMM_F32_ERR_BAD_KERNEL;
  return run_entry(t[index], op, r.p, r.dev, s);
}

const char* selected_impl(const Op& op, int64_t M, int64_t N, int64_t K, int64_t lda,
                          int64_t ldb, int64_t ldc, const void* A, const void* B) {
  const int64_t kMax = GEMM_F32_MAX_DIM;
  if (M < 0 || N < 0 || K < 0 || M > kMax || N > kMax || K > kMax) return "invalid";
  const int64_t a_cols = op.ta ? M : K, b_cols = op.tb ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return "invalid";
  const std::string name = select_name(op, M, N, K, lda, ldb, A, B);
  if (name == "empty") return "empty";
  if (name == "fill_zero_k0") return "fill_zero_k0";
  const int idx = find_entry(name);
  return idx < 0 ? "invalid" : entries()[idx].name.c_str();
}

// ---- strided batch ---------------------------------------------------------
// Product b reads A + b*sa (M x K, pitch lda) and B + b*sb (K x N, pitch ldb)
// and writes C + b*sc (M x N, pitch ldc).  Strides of A and B may be 0 (one
// matrix shared by every product); C's windows must not overlap.
struct Batch {
  int64_t sa = 0, sb = 0, sc = 0, count = 1;
};

// Byte extent of a pitched matrix (rows x cols, pitch ld), 0 if empty.
uint64_t extent_bytes(int64_t rows, int64_t cols, int64_t ld) {
  return rows > 0 && cols > 0 ? (uint64_t)(((rows - 1) * ld + cols) * 4) : 0;
}

int check_batch(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, const float* C, int64_t ldc, const Batch& bt) {
  if (bt.count < 0 || bt.count > GEMM_F32_MAX_DIM) return GEMM_F32_ERR_INVALID_DIM;
  // dimensions, pitches, NULL pointers and alignment of the first product
  int rc = check_args(Op{}, M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMM_F32_OK || bt.count <= 1) return rc;
  if (bt.sa < 0 || bt.sb < 0 || bt.sc < 0) return GEMM_F32_ERR_INVALID_LD;
  const int64_t kMaxElems = INT64_C(1) << 60;
  const int64_t last = bt.count - 1;
  if (bt.sa > kMaxElems / last || bt.sb > kMaxElems / last || bt.sc > kMaxElems / last)
    return GEMM_F32_ERR_INVALID_LD;
  const uint64_t ea = extent_bytes(M, K, lda), eb = extent_bytes(K, N, ldb),
                 ec = extent_bytes(M, N, ldc);
  if (ec == 0) return GEMM_F32_OK;   // nothing is written
  // the products' C windows must not overlap one another ...
  if ((uint64_t)bt.sc * 4 < ec) return GEMM_F32_ERR_ALIAS;
  // ... nor any A or B of the batch (whole address ranges)
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)(last * bt.sc * 4) + ec;
  if (ea) {
    const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)(last * bt.sa * 4) + ea;
    if (c0 < a1 && a0 < c1) return GEMM_F32_ERR_ALIAS;
  }
  if (eb) {
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(last * bt.sb * 4) + eb;
    if (c0 < b1 && b0 < c1) return GEMM_F32_ERR_ALIAS;
  }
  return GEMM_F32_OK;
}

// Kernel for a batch of more than one product: the first row of the plain
// table whose kernel takes a whole batch (the whole-K MFMA kernels; no K
// split, no skinny kernel) and these arguments, sized by all tiles of the
// batch.  A direct-to-LDS kernel also needs every product 16-byte aligned.
std::string select_name_batched(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                                const void* A, const void* B, const Batch& bt) {
  if (bt.count <= 1) return select_name(Op{}, M, N, K, lda, ldb, A, B);
  if (M == 0 || N == 0) return "empty";
  if (K == 0) return "fill_zero_k0";
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128) * bt.count;
  for (const auto& row : gemmf32::kTuningGfx950) {
    if (M > row.max_m || tiles < row.min_tiles) continue;
    if (row.max_tiles > 0 && tiles > row.max_tiles) continue;
    const int idx = find_entry(row.kernel);
    if (idx < 0 || entries()[idx].kind != Kind::Mfma) continue;
    if (!accepts(entries()[idx], Op{}, M, N, K, lda, ldb, A, B)) continue;
    if (gemmf32::mfma_variant(entries()[idx].sub).lds_dma && (bt.sa % 4 != 0 || bt.sb % 4 != 0))
      continue;
    if (row.wave_slots > 0 && !fills_waves(entries()[idx], M, N, bt.count, row.wave_slots))
      continue;
    return row.kernel;
  }
  // the rows above always end in a kernel that takes any operands
  return "ref_naive";
}

int gemm_batched_impl(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float* C, int64_t ldc, const Batch& bt,
                      void* stream) {
  int rc = check_batch(M, N, K, A, lda, B, ldb, C, ldc, bt);
  if (rc != GEMM_F32_OK) return rc;
  if (bt.count == 0 || M == 0 || N == 0) return GEMM_F32_OK;
  if (bt.count == 1) return gemm_impl(Op{}, M, N, K, A, lda, B, ldb, C, ldc, stream);
  Prepared r = prepare(Op{}, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK) return r.status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int idx = -1;
  if (K > 0) {
    idx = find_entry(select_name_batched(M, N, K, lda, ldb, A, B, bt));
    if (idx < 0) return GEMM_F32_ERR_BAD_KERNEL;
  }
  // launches of at most kMaxLaunchBatch products (grid z)
  for (int64_t b0 = 0; b0 < bt.count; b0 += gemmf32::kMaxLaunchBatch) {
    Problem q = r.p;
    q.A += b0 * bt.sa;
    q.B += b0 * bt.sb;
    q.C += b0 * bt.sc;
    q.sa = bt.sa;
    q.sb = bt.sb;
    q.sc = bt.sc;
    const int64_t n = bt.count - b0;
    q.batch = (int)(n < gemmf32::kMaxLaunchBatch ? n : gemmf32::kMaxLaunchBatch);
    rc = K == 0 ? run_k0(Op{}, q, s) : run_entry(entries()[idx], Op{}, q, r.dev, s);
    if (rc != GEMM_F32_OK) return rc;
  }
  return GEMM_F32_OK;
}

Op make_op(int transA, int transB, float alpha, float beta, const float* bias = nullptr,
           int act = 0) {
  Op op;
  op.ta = transA != 0;
  op.tb = transB != 0;
  op.alpha = alpha;
  op.beta = beta;
  op.bias = bias;
  op.act = act;
  return op;
}

}  // namespace

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
             int64_t ldb, float* C, int64_t ldc, void* stream) {
  return gemm_impl(Op{}, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_noalloc(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                     const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  return gemm_noalloc_impl(M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                int64_t ldc, void* stream) {
  return gemm_impl(make_op(transA, transB, alpha, beta), M, N, K, A, lda, B, ldb, C, ldc,
                   stream);
}

int gemm_f32_fused(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                   const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                   float* C, int64_t ldc, const float* bias, int activation, void* stream) {
  return gemm_impl(make_op(transA, transB, alpha, beta, bias, activation), M, N, K, A, lda, B,
                   ldb, C, ldc, stream);
}

int gemm_f32_run_kernel_fused(int index, int transA, int transB, int64_t M, int64_t N,
                              int64_t K, float alpha, const float* A, int64_t lda,
                              const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
                              const float* bias, int activation, void* stream) {
  return run_kernel_impl(index, make_op(transA, transB, alpha, beta, bias, activation), M, N, K,
                         A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_batched(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                     int64_t strideA, const float* B, int64_t ldb, int64_t strideB, float* C,
                     int64_t ldc, int64_t strideC, int64_t batch, void* stream) {
  Batch bt;
  bt.sa = strideA;
  bt.sb = strideB;
  bt.sc = strideC;
  bt.count = batch;
  return gemm_batched_impl(M, N, K, A, lda, B, ldb, C, ldc, bt, stream);
}

const char* gemm_f32_selected_kernel_batched(int64_t M, int64_t N, int64_t K, int64_t lda,
                                             int64_t strideA, int64_t ldb, int64_t strideB,
                                             int64_t ldc, int64_t batch, const void* A,
                                             const void* B) {
  if (batch < 0 || batch > GEMM_F32_MAX_DIM || strideA < 0 || strideB < 0) return "invalid";
  if (batch <= 1) return selected_impl(Op{}, M, N, K, lda, ldb, ldc, A, B);
  const char* plain = selected_impl(Op{}, M, N, K, lda, ldb, ldc, A, B);
  if (std::strcmp(plain, "invalid") == 0) return plain;
  Batch bt;
  bt.sa = strideA;
  bt.sb = strideB;
  bt.count = batch;
  const std::string name = select_name_batched(M, N, K, lda, ldb, A, B, bt);
  if (name == "empty") return "empty";
  if (name == "fill_zero_k0") return "fill_zero_k0";
  const int idx = find_entry(name);
  return idx < 0 ? "invalid" : entries()[idx].name.c_str();
}

int reduce_sum_f32(int64_t n, const float* x, float* out, void* stream) {
  if (n < 0 || n > (INT64_C(1) << 60)) return GEMM_F32_ERR_INVALID_DIM;
  if ((n > 0 && !x) || !out) return GEMM_F32_ERR_NULL_PTR;
  if ((n > 0 && !aligned4(x)) || !aligned4(out)) return GEMM_F32_ERR_POINTER;
  if (n > 0) {
    const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)(n * 4), o = (uintptr_t)out;
    if (o + 4 > x0 && o < x1) return GEMM_F32_ERR_ALIAS;
  }
  int dev = -1;
  int rc = check_device(&dev);
  if (rc != GEMM_F32_OK) return rc;
  if (n > 0 && (rc = check_pointer(x, dev)) != GEMM_F32_OK) return rc;
  if ((rc = check_pointer(out, dev)) != GEMM_F32_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const gemmf32::ReducePlan pl = gemmf32::plan_reduce(n);
  unsigned long long* slots = nullptr;
  if (pl.groups > 1 &&
      (rc = get_exchange_slots(dev, s, (size_t)pl.groups, &slots)) != GEMM_F32_OK)
    return rc;
  if (gemmf32::launch_reduce_sum(n, x, out, slots, s) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

int gemm_f32_ref_gpu(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                     const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  const Op op;
  Prepared r = prepare(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK || M == 0 || N == 0) return r.status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      K == 0 ? gemmf32::launch_scale(r.p, gemmf32::Epilogue{}, s) : gemmf32::launch_ref(r.p, s);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

int gemm_f32_run_kernel(int index, int64_t M, int64_t N, int64_t K, const float* A,
                        int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                        void* stream) {
  return run_kernel_impl(index, Op{}, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_run_kernel_ex(int index, int transA, int transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const float* A, int64_t lda, const float* B,
                           int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
  return run_kernel_impl(index, make_op(transA, transB, alpha, beta), M, N, K, A, lda, B, ldb,
                         C, ldc, stream);
}

int gemm_f32_clock_probe(int64_t iters, unsigned long long* stamps, int* wall_khz,
                         int* max_khz, void* stream) {
  static_assert(GEMM_F32_CLOCK_PROBE_WORKGROUPS == gemmf32::kClockProbeWorkgroups,
                "one probe grid size");
  if (iters < 1 || iters > (INT64_C(1) << 24)) return GEMM_F32_ERR_INVALID_DIM;
  if (!stamps) return GEMM_F32_ERR_NULL_PTR;
  if (((uintptr_t)stamps & 7u) != 0) return GEMM_F32_ERR_POINTER;
  int dev = -1;
  int rc = check_device(&dev);
  if (rc != GEMM_F32_OK) return rc;
  if ((rc = check_pointer(stamps, dev)) != GEMM_F32_OK) return rc;
  if ((wall_khz &&
       hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) ||
      (max_khz && hipDeviceGetAttribute(max_khz, hipDeviceAttributeClockRate, dev) != hipSuccess)) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_DEVICE;
  }
  if (gemmf32::launch_clock_probe((int)iters, stamps, static_cast<hipStream_t>(stream)) !=
      hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

const char* gemm_f32_status_string(int status) {
  switch (status) {
    case GEMM_F32_OK: return "ok";
    case GEMM_F32_ERR_INVALID_DIM: return "invalid dimension (M, N or K negative or above GEMM_F32_MAX_DIM)";
    case GEMM_F32_ERR_INVALID_LD: return "invalid leading dimension (pitch below row length)";
    case GEMM_F32_ERR_NULL_PTR: return "null pointer for a non-empty matrix";
    case GEMM_F32_ERR_ALIAS: return "C overlaps A or B";
    case GEMM_F32_ERR_DEVICE: return "no usable HIP device, or the current device is not gfx950";
    case GEMM_F32_ERR_WORKSPACE: return "workspace allocation failed";
    case GEMM_F32_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_F32_ERR_BAD_KERNEL: return "kernel index unknown or unable to run these arguments";
    case GEMM_F32_ERR_POINTER: return "pointer is not device memory the current device can access";
    case GEMM_F32_ERR_INVALID_ARG: return "unknown activation";
    case GEMM_F32_ERR_SCRATCH: return "the call needs more scratch than gemm_f32_noalloc's fixed array holds";
    default: return "unknown status";
  }
}

const char* gemm_f32_selected_kernel(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                                     int64_t ldc, const void* A, const void* B, const void* C) {
  (void)C;
  return selected_impl(Op{}, M, N, K, lda, ldb, ldc, A, B);
}

const char* gemm_f32_selected_kernel_ex(int transA, int transB, int64_t M, int64_t N, int64_t K,
                                        int64_t lda, int64_t ldb, int64_t ldc, float alpha,
                                        float beta, const void* A, const void* B,
                                        const void* C) {
  (void)C;
  return selected_impl(make_op(transA, transB, alpha, beta), M, N, K, lda, ldb, ldc, A, B);
}

int gemm_f32_version(void) { return GEMM_F32_VERSION; }

int gemm_f32_kernel_count(void) { return (int)entries().size(); }

const char* gemm_f32_kernel_name(int index) {
  const auto& t = entries();
  if (index < 0 || index >= (int)t.size()) return nullptr;
  return t[index].name.c_str();
}

int gemm_f32_release_workspaces(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int rc = GEMM_F32_OK;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto* m : {g_ws, g_xs}) {
    if (!m) continue;
    for (auto& kv : *m) {
      Workspace& w = kv.second;
      if (w.ptr) w.retired.push_back(w.ptr);
      if (w.retired.empty()) continue;
      if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        rc = GEMM_F32_ERR_WORKSPACE;
        continue;
      }
      for (void* p : w.retired) {
        if (hipFree(p) != hipSuccess) {
          (void)hipGetLastError();
          rc = GEMM_F32_ERR_WORKSPACE;
        }
      }
    }
    m->clear();
  }
  if (have_cur) (void)hipSetDevice(cur);
  return rc;
}

#if GEMM_F32_SWEEP
int gemm_f32_stamped(int index, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                     const float* B, int64_t ldb, float* C, int64_t ldc,
                     unsigned long long* stamps, int64_t stamp_words, void* stream) {
  const auto& t = entries();
  if (index < 0 || index >= (int)t.size() || t[index].kind != Kind::Mfma)
    return GEMM_F32_ERR_BAD_KERNEL;
  // the entry's tile among the direct-to-LDS ones
  int tile = -1;
  for (int i = 0; i < gemmf32::mfma_dma_variant_count(); ++i)
    if (t[index].name == gemmf32::mfma_dma_variant(i).name) tile = i;
  if (tile < 0) return GEMM_F32_ERR_BAD_KERNEL;
  const Op op;
  Prepared r = prepare(op, M, N, K, A, lda, B, ldb, C, ldc);
  if (r.status != GEMM_F32_OK) return r.status;
  if (M == 0 || N == 0 || K == 0 || !entry_accepts(t[index], op, r.p))
    return GEMM_F32_ERR_BAD_KERNEL;
  const auto& v = gemmf32::mfma_dma_variant(tile);
  const int64_t tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
  if (!stamps) return GEMM_F32_ERR_NULL_PTR;
  if (((uintptr_t)stamps & 7u) != 0) return GEMM_F32_ERR_POINTER;
  if (stamp_words < 6 * tiles) return GEMM_F32_ERR_INVALID_DIM;
  int rc = check_pointer(stamps, r.dev);
  if (rc != GEMM_F32_OK) return rc;
  if (gemmf32::launch_dma_stamped(tile, r.p, op.epilogue(), stamps, stamp_words,
                                  static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}

int gemm_f32_read_probe(const float* x, int64_t n, int groups, float* out, void* stream) {
  if (groups < 1 || groups > 65535 || n <= 0 || n > (INT64_C(1) << 40) ||
      n % ((int64_t)256 * groups) != 0)
    return GEMM_F32_ERR_INVALID_DIM;
  if (!x || !out) return GEMM_F32_ERR_NULL_PTR;
  if (((uintptr_t)x & 15u) != 0 || !aligned4(out)) return GEMM_F32_ERR_POINTER;
  const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)(n * 4), o = (uintptr_t)out;
  if (o + (uintptr_t)groups * 32 > x0 && o < x1) return GEMM_F32_ERR_ALIAS;
  int dev = -1;
  int rc = check_device(&dev);
  if (rc != GEMM_F32_OK) return rc;
  if ((rc = check_pointer(x, dev)) != GEMM_F32_OK || (rc = check_pointer(out, dev)) != GEMM_F32_OK)
    return rc;
  if (gemmf32::launch_read_probe(x, n, groups, out, static_cast<hipStream_t>(stream)) !=
      hipSuccess) {
    (void)hipGetLastError();
    return GEMM_F32_ERR_LAUNCH;
  }
  return GEMM_F32_OK;
}
#endif

}  // extern "C"
