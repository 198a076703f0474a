"""The C ABI on the host: the library loads, exports what the header
declares, and rejects bad arguments before touching any device.  CPU only:
no call here reaches a kernel launch."""
import ctypes
import re
from pathlib import Path

import pytest

from dense_fp32_gemm_f32_amd import binding

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "gemm_f32.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gemm|reduce_sum)_f32\w*)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("gemm_f32", "gemm_f32_ref_gpu", "gemm_f32_status_string",
                 "gemm_f32_selected_kernel", "gemm_f32_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in gemm_f32.h but not exported"
    assert sorted(binding.EXPORTS) == declared_functions()


SWEEP_HEADER = ROOT / "include" / "gemm_f32_sweep.h"


def sweep_only_functions():
    text = re.sub(r"/\*.*?\*/", "", SWEEP_HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f32\w*)\s*\(", text)))


def test_sweep_only_calls_stay_out_of_the_product_library():
    lib = binding.load()
    assert sweep_only_functions() == ["gemm_f32_read_probe", "gemm_f32_stamped"]
    for name in sweep_only_functions():
        assert not hasattr(lib, name), f"{name} is for the sweep build only"


def test_sweep_library_exports_both_headers():
    from dense_fp32_gemm_f32_amd import build_lib
    if not build_lib.SWEEP_LIB.exists():
        pytest.skip("the sweep library is not built")
    lib = ctypes.CDLL(str(build_lib.SWEEP_LIB))
    for name in declared_functions() + sweep_only_functions():
        assert hasattr(lib, name), f"{name} not exported by the sweep library"
    # an entry that is not a direct-to-LDS tile is refused before any device call
    lib.gemm_f32_stamped.argtypes = [ctypes.c_int] + [ctypes.c_int64] * 3 + [
        ctypes.c_void_p, ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.gemm_f32_kernel_count.restype = ctypes.c_int
    lib.gemm_f32_kernel_name.argtypes = [ctypes.c_int]
    lib.gemm_f32_kernel_name.restype = ctypes.c_char_p
    names = [lib.gemm_f32_kernel_name(i).decode() for i in range(lib.gemm_f32_kernel_count())]
    other = names.index("ref_naive")
    assert lib.gemm_f32_stamped(other, 64, 64, 64, P16, 64, Q16, 64, R16, 64, P16, 96, None) == 8
    assert lib.gemm_f32_stamped(len(names), 64, 64, 64, P16, 64, Q16, 64, R16, 64, P16, 96,
                                None) == 8
    # the read probe's argument errors, before any device call
    lib.gemm_f32_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    probe = lib.gemm_f32_read_probe
    assert probe(P16, 1 << 20, 0, Q16, None) == 1          # no workgroup
    assert probe(P16, 1 << 20, 65536, Q16, None) == 1      # too many
    assert probe(P16, 0, 1, Q16, None) == 1                # empty
    assert probe(P16, (1 << 20) + 64, 4, Q16, None) == 1   # not whole 1 KiB pieces per group
    assert probe(None, 1 << 20, 4, Q16, None) == 3
    assert probe(P16, 1 << 20, 4, None, None) == 3
    assert probe(P16 + 4, 1 << 20, 4, Q16, None) == 9      # x not 16-byte aligned
    assert probe(P16, 1 << 20, 4, P16 + 64, None) == 4     # out inside x


def test_version():
    assert binding.gemm_f32_version() == 5


def test_status_strings():
    for code in list(binding.STATUS_NAMES) + [1234]:
        s = binding.gemm_f32_status_string(code)
        assert isinstance(s, str) and s
    assert binding.gemm_f32_status_string(0) == "ok"


def test_kernel_table():
    names = binding.kernel_names()
    assert len(names) == len(set(names)) == binding.gemm_f32_kernel_count()
    assert any(n.startswith("mfma_") for n in names)
    assert any(n.startswith("skinny") for n in names)
    assert "ref_naive" in names
    assert binding.gemm_f32_kernel_name(-1) is None
    assert binding.gemm_f32_kernel_name(len(names)) is None


# Pointers that are never dereferenced: these calls fail validation first.
P16 = 0x10000
Q16 = 0x90000000
R16 = 0x190000000


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, P16, 4, Q16, 4, R16, 4), 1),
    ((4, -1, 4, P16, 4, Q16, 4, R16, 4), 1),
    ((4, 4, -1, P16, 4, Q16, 4, R16, 4), 1),
    ((2 ** 31 - 2 ** 16 + 1, 4, 4, P16, 4, Q16, 4, R16, 4), 1),
    ((4, 4, 4, P16, 3, Q16, 4, R16, 4), 2),
    ((4, 4, 4, P16, 4, Q16, 3, R16, 4), 2),
    ((4, 4, 4, P16, 4, Q16, 4, R16, 3), 2),
    ((4, 4, 0, P16, 0, Q16, 4, R16, 4), 2),
    ((4, 4, 4, 0, 4, Q16, 4, R16, 4), 3),
    ((4, 4, 4, P16, 4, 0, 4, R16, 4), 3),
    ((4, 4, 4, P16, 4, Q16, 4, 0, 4), 3),
    ((4, 4, 4, P16, 4, Q16, 4, P16 + 8, 4), 4),
    ((4, 4, 4, P16, 4, Q16, 4, Q16 + 60, 4), 4),
])
def test_argument_errors_before_any_device_call(args, code):
    assert binding.gemm_f32(*args, 0) == code
    assert binding.gemm_f32_ref_gpu(*args, 0) == code
    assert binding.gemm_f32_noalloc(*args, 0) == code
    assert binding.gemm_f32_run_kernel(0, *args, 0) == code


def test_empty_problems_succeed_without_a_device():
    assert binding.gemm_f32(0, 4, 4, 0, 4, Q16, 4, 0, 4, 0) == 0
    assert binding.gemm_f32(4, 0, 4, P16, 4, 0, 1, 0, 1, 0) == 0
    assert binding.gemm_f32_noalloc(0, 4, 4, 0, 4, Q16, 4, 0, 4, 0) == 0
    # a NULL A is fine when A has no elements, even if M > 0 (K == 0), but the
    # K == 0 fill needs a device, so only the M == 0 / N == 0 cases run here


def test_adjacent_but_not_overlapping_is_not_alias():
    # C starts right after A's last element: validation passes, then the
    # device check (no GPU here, or a real one) decides; never ERR_ALIAS.
    rc = binding.gemm_f32(4, 4, 4, P16, 4, Q16, 4, P16 + 64, 4, 0)
    assert rc != 4


@pytest.mark.parametrize("M,N,K,lda,ldb,A,B,expect", [
    (0, 5, 5, 5, 5, P16, Q16, "empty"),
    (5, 0, 5, 5, 1, P16, Q16, "empty"),
    (5, 5, 0, 1, 5, P16, Q16, "fill_zero_k0"),
    (8, 8192, 8192, 8192, 8192, P16, Q16, "skinnyx_w8_c2_u2"),
    (3, 8192, 8192, 8192, 8192, P16, Q16, "skinnyx_w8_c2_u2"),
    (16, 4096, 4096, 4096, 4096, P16, Q16, "skinnyx_w8_c2_u2"),
    (8, 3001, 1531, 1531, 3001, P16, Q16, "skinnyx_w8_c2_u2"),
    # up to 2048 columns (16 tiles of 128): 16 waves per workgroup
    (8, 1024, 8192, 8192, 1024, P16, Q16, "skinnyx_w16_c2_u2"),
    (16, 2048, 8192, 8192, 2048, P16, Q16, "skinnyx_w16_c2_u2"),
    (1, 7, 5, 5, 7, P16, Q16, "skinnyx_w16_c2_u2"),
    (8, 2049, 8192, 8192, 2049, P16, Q16, "skinnyx_w8_c2_u2"),
    # wide N: KiB row runs, when B's rows are 16-byte aligned; else the tile kernel
    (8, 28672, 4096, 4096, 28672, P16, Q16, "skinnyr_c2_r4"),
    (8, 28672, 4096, 4096, 28673, P16, Q16, "skinnyx_w8_c2_u2"),
    (16, 28672, 4096, 4096, 28672, P16, Q16, "skinnyx_w8_c2_u2"),
    (4096, 4096, 4096, 4096, 4096, P16, Q16, "mfma_256x256x32_w64x128_d6"),
    # 256 x 256 tiles only where they fill whole waves of the 256 CUs
    (8192, 8192, 4096, 4096, 8192, P16, Q16, "mfma_256x256x32_w64x128_d6"),
    (6144, 6144, 4096, 4096, 6144, P16, Q16, "mfma_128x256x16_w64x128_d6"),
    # operands the 16-byte direct loads cannot take: 64 x 64 tiles copied
    # into LDS one float per lane
    (4096, 4097, 4096, 4096, 4097, P16, Q16, "mfma_64x64x16_w32x32_d4"),
    (8191, 8191, 2001, 2001, 8191, P16, Q16, "mfma_64x64x16_w32x32_d4"),
    (2047, 3001, 1531, 1531, 3001, P16, Q16, "mfma_64x64x16_w32x32_d4"),
    (3001, 2047, 1531, 1531, 2047, P16, Q16, "mfma_64x64x16_w32x32_d4"),
    (2047, 3001, 32, 32, 3001, P16, Q16, "mfma_64x64x16_w32x32_d4"),
    (767, 769, 771, 771, 769, P16, Q16, "mfma_64x64x32_w32x32_d4"),
    # ... unless K is below two K-tiles or a tile's offsets exceed 32 bits:
    # the register-staged tile whose grid leaves its last wave at least 90 %
    # full (or makes 4+ waves)
    (4096, 4097, 31, 31, 4097, P16, Q16, "mfma_128x192x32_w32x96_p5"),      # 704 of 768
    (8191, 8191, 31, 31, 8191, P16, Q16, "mfma_128x128x32_w64x64_p5"),      # 8 waves of 512
    (6001, 6001, 999, 2 ** 23 + 1, 6001, P16, Q16, "mfma_128x128x32_w64x64_p5"),  # 4.3 waves
    (2047, 3001, 31, 31, 3001, P16, Q16, "mfma_128x192x32_w32x96_p5"),      # 256 tiles
    (3001, 2047, 31, 31, 2047, P16, Q16, "mfma_192x128x32_w96x32_p5"),      # 256 tiles
    (2049, 2049, 31, 31, 2049, P16, Q16, "mfma_64x64x32_w32x32_p5"),        # 187 of 256
    (767, 769, 63, 63, 769, P16, Q16, "mfma_64x64x32_w32x32_p5"),
    (7936, 7936, 4096, 4096, 7936, P16, Q16, "mfma_256x256x32_w64x128_d6"),  # 961 of 1024
    # aligned operands: 128 x 192 (or 192 x 128) direct-to-LDS tiles where one
    # per CU fills whole waves, else 128 x 128
    (2048, 3072, 1536, 1536, 3072, P16, Q16, "mfma_128x192x32_w32x96_d6"),   # 256 tiles
    (3072, 2048, 1536, 1536, 2048, P16, Q16, "mfma_192x128x32_w96x32_d6"),   # 256 tiles
    (2048, 3008, 1536, 1536, 3008, P16, Q16, "mfma_128x192x32_w32x96_d6"),   # 256 tiles
    (2048, 2048, 2048, 2048, 2048, P16, Q16, "mfma_128x128x32_w64x32_d6"),   # 176 of 256
    (2048, 2048, 2064, 2064, 2048, P16, Q16, "mfma_128x128x16_w64x64_d6"),   # K % 32 = 16
    (512, 512, 512, 512, 512, P16, Q16, "mfma_32x32x8_k4_g4_small"),
    (768, 768, 768, 768, 768, P16, Q16, "mfma_64x64x32_w32x32_d6"),
    (1024, 1024, 1024, 1024, 1024, P16, Q16, "mfma_64x64x32_w32x32_d6"),
])
def test_dispatcher_families(M, N, K, lda, ldb, A, B, expect):
    name = binding.gemm_f32_selected_kernel(M, N, K, lda, ldb, max(N, 1), A, B, R16)
    assert name.startswith(expect), name


def test_dispatcher_picks_128_bit_loads_for_any_pitch():
    """128-bit loads need only 4-byte aligned rows, so every accepted call gets
    the table's preferred load widths whatever its pitches."""
    sel = binding.gemm_f32_selected_kernel
    names = binding.kernel_names()
    for args in [(4096, 4096, 4096, 4096, 4096, 4096), (4096, 4096, 4096, 4097, 4096, 4096),
                 (4096, 4096, 4096, 4096, 4098, 4096), (1000, 999, 777, 777, 999, 999),
                 (8, 8192, 8192, 8192, 8192, 8192), (1, 100, 100, 101, 100, 100),
                 (16, 64, 64, 64, 64, 64), (17, 64, 64, 64, 64, 64), (300, 40, 50, 50, 40, 40),
                 (2047, 3001, 1531, 1531, 3001, 3001), (8, 3001, 1531, 1531, 3001, 3001)]:
        M, N, K, lda, ldb, ldc = args
        for pa, pb in [(P16, Q16), (P16 + 4, Q16), (P16, Q16 + 8), (P16 + 4, Q16 + 12)]:
            name = sel(M, N, K, lda, ldb, ldc, pa, pb, R16)
            assert name in names, name
            assert not name.endswith("_scalar"), name



def test_direct_to_lds_kernels_only_for_aligned_operands():
    """Kernels with direct-to-LDS loads need 16-byte aligned A and B, lda, ldb
    and N multiples of 4 and K a multiple of their K-tile; otherwise the
    dispatcher takes the register-staged kernel of the same shape class."""
    sel = binding.gemm_f32_selected_kernel
    assert "_d6_" in sel(4096, 4096, 4096, 4096, 4096, 4096, P16, Q16, R16)
    assert "_d6_" in sel(1024, 1024, 1024, 1024, 1024, 1024, P16, Q16, R16)
    assert "_d6_" in sel(768, 768, 768, 768, 768, 768, P16, Q16, R16)
    for args in [(4096, 4096, 4096, 4097, 4096, 4096, P16, Q16),      # lda % 4
                 (4096, 4096, 4096, 4096, 4098, 4096, P16, Q16),      # ldb % 4
                 (4096, 4095, 4096, 4096, 4096, 4096, P16, Q16),      # N % 4
                 (4096, 4096, 4100, 4100, 4096, 4096, P16, Q16),      # K % 16
                 (4096, 4096, 4096, 4096, 4096, 4096, P16 + 4, Q16),  # A 4-byte aligned
                 (4096, 4096, 4096, 4096, 4096, 4096, P16, Q16 + 8)]: # B 8-byte aligned
        M, N, K, lda, ldb, ldc, pa, pb = args
        name = sel(M, N, K, lda, ldb, ldc, pa, pb, R16)
        assert name.startswith("mfma_") and "_d6_" not in name, (args, name)


def test_misaligned_pointers_are_rejected():
    assert binding.gemm_f32(4, 4, 4, P16 + 2, 4, Q16, 4, R16, 4, 0) == 9
    assert binding.gemm_f32(4, 4, 4, P16, 4, Q16 + 1, 4, R16, 4, 0) == 9
    assert binding.gemm_f32(4, 4, 4, P16, 4, Q16, 4, R16 + 3, 4, 0) == 9


def test_dispatcher_rejects_bad_arguments():
    sel = binding.gemm_f32_selected_kernel
    assert sel(-1, 4, 4, 4, 4, 4, P16, Q16, R16) == "invalid"
    assert sel(4, 4, 4, 3, 4, 4, P16, Q16, R16) == "invalid"


def _tuning_table_names():
    """Every kernel name the gfx950 tuning tables can select, read from the
    header: the plain and skinny rows as written, the extended-operation rows
    with each transposed layout's suffix."""
    import re
    text = (ROOT / "dense_fp32_gemm_f32_amd" / "csrc" / "tuning_gfx950.h").read_text()

    def rows(table):
        body = text[text.index(table):]
        body = body[:body.index("};")]
        return re.findall(r'^\s*\{[^"]*"([a-z0-9_]+)"', body, re.M)
    names = set(rows("kTuningGfx950[] = {")) | set(rows("kTuningGfx950Skinny[] = {"))
    for prefix in rows("kTuningGfx950Ex[] = {"):
        names |= {prefix + lay for lay in ("_nt", "_tn", "_tt")}
    return names


def test_default_table_is_what_the_tuning_tables_select():
    """The default build holds every kernel a tuning row names, the reference
    kernel, and nothing else (sweep-only variants need GEMM_F32_SWEEP)."""
    names = set(binding.kernel_names())
    wanted = _tuning_table_names()
    assert len(wanted) > 20
    assert wanted <= names, sorted(wanted - names)
    assert names - wanted == {"ref_naive"}, sorted(names - wanted)


# ---- the extended operation (gemm_f32_ex) -------------------------------------

LAYOUTS = {(0, 0): "_nn", (0, 1): "_nt", (1, 0): "_tn", (1, 1): "_tt"}


@pytest.mark.parametrize("ta,tb", list(LAYOUTS))
def test_ex_dispatcher_picks_the_layout_kernel(ta, tb):
    sel = binding.gemm_f32_selected_kernel_ex
    names = binding.kernel_names()
    for (M, N, K) in [(4096, 4096, 4096), (2047, 3001, 1531), (512, 512, 512), (8, 8192, 8192),
                      (1, 3, 5)]:
        lda = M if ta else K
        ldb = K if tb else N
        name = sel(ta, tb, M, N, K, lda, ldb, N, 1.5, 0.5, P16, Q16, R16)
        assert name in names, name
        if M <= 16:
            assert name.startswith("skinny"), name
            if (ta, tb) != (0, 0):
                assert name.endswith(LAYOUTS[(ta, tb)]), name
        elif (ta, tb) == (0, 0):
            # A and B as stored: the plain table's kernel, which applies the epilogue
            assert name == binding.gemm_f32_selected_kernel(M, N, K, lda, ldb, N, P16, Q16,
                                                            R16), name
        else:
            assert name.startswith("mfmaex_") and name.endswith(LAYOUTS[(ta, tb)]), name


def test_ex_plain_case_runs_what_gemm_f32_runs():
    for (M, N, K) in [(4096, 4096, 4096), (2047, 3001, 1531), (512, 512, 512), (8, 8192, 8192)]:
        plain = binding.gemm_f32_selected_kernel(M, N, K, K, N, N, P16, Q16, R16)
        ex = binding.gemm_f32_selected_kernel_ex(0, 0, M, N, K, K, N, N, 1.0, 0.0, P16, Q16, R16)
        assert plain == ex
        # alpha or beta other than 1, 0 with A and B as stored: the same kernel,
        # whose store applies the epilogue
        name = binding.gemm_f32_selected_kernel_ex(0, 0, M, N, K, K, N, N, 2.0, 0.5, P16, Q16,
                                                   R16)
        assert name == plain, (name, plain)


def test_ex_pitches_are_checked_against_the_stored_shapes():
    f = binding.gemm_f32_ex
    # A stored K x M when transposed: lda must cover M, not K
    assert f(1, 0, 100, 50, 30, 1.0, P16, 30, Q16, 50, 0.0, R16, 50, 0) == 2
    # B stored N x K when transposed: ldb must cover K
    assert f(0, 1, 100, 50, 30, 1.0, P16, 30, Q16, 29, 0.0, R16, 50, 0) == 2
    assert f(0, 1, 100, 50, 30, 1.0, P16, 30, Q16, 50, 0.0, R16, 49, 0) == 2
    assert f(0, 0, -1, 50, 30, 1.0, P16, 30, Q16, 50, 0.0, R16, 50, 0) == 1
    assert f(1, 1, 100, 50, 30, 1.0, 0, 100, Q16, 30, 0.0, R16, 50, 0) == 3


def test_ex_alias_uses_the_stored_extent():
    f = binding.gemm_f32_ex
    # A stored 30 x 100 (transposed) ends 12000 bytes after P16; C right after is fine,
    # C inside it is not
    assert f(1, 0, 100, 50, 30, 1.0, P16, 100, Q16, 50, 0.0, P16 + 11996, 50, 0) == 4


def test_kernel_names_are_unique():
    names = binding.kernel_names()
    assert len(names) == len(set(names)), [n for n in names if names.count(n) > 1][:5]


# ---- strided batch (gemm_f32_batched) -------------------------------------------

def _batched(M, N, K, A, lda, sa, B, ldb, sb, C, ldc, sc, batch):
    return binding.gemm_f32_batched(M, N, K, A, lda, sa, B, ldb, sb, C, ldc, sc, batch, 0)


def test_batched_argument_errors_before_any_device_call():
    big = 1 << 28
    # negative batch; negative strides
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, 16, R16, 4, 16, -1) == 1
    assert _batched(4, 4, 4, P16, 4, -16, Q16, 4, 16, R16, 4, 16, 2) == 2
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, -16, R16, 4, 16, 2) == 2
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, 16, R16, 4, -16, 2) == 2
    # the per-product checks still apply
    assert _batched(4, 4, 4, P16, 3, 16, Q16, 4, 16, R16, 4, 16, 2) == 2
    assert _batched(4, 4, 4, 0, 4, 16, Q16, 4, 16, R16, 4, 16, 2) == 3
    # C windows of two products overlap (stride shorter than one window)
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, 16, R16, 4, 15, 2) == 4
    # the second product's C runs into the batch of A (A stride 0 is fine)
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, 0, P16 + 4 * 16 * 4, 4, 16, 8) == 4
    # strides too large for 64-bit extents
    assert _batched(4, 4, 4, P16, 4, big * big, Q16, 4, 16, R16, 4, 16, 1 << 20) == 2


def test_batched_empty_and_single():
    # batch 0, M or N 0: successful no-ops with no device
    assert _batched(4, 4, 4, P16, 4, 16, Q16, 4, 16, R16, 4, 16, 0) == 0
    assert _batched(0, 4, 4, P16, 4, 16, Q16, 4, 16, R16, 4, 16, 3) == 0
    assert _batched(4, 0, 4, P16, 4, 16, Q16, 1, 16, R16, 1, 16, 3) == 0


def test_batched_selection():
    sel = binding.gemm_f32_selected_kernel_batched
    names = binding.kernel_names()
    # batch 1 is gemm_f32
    for (M, N, K) in [(4096, 4096, 4096), (8, 8192, 8192), (512, 512, 512)]:
        assert sel(M, N, K, K, M * K, N, K * N, N, 1, P16, Q16) == \
            binding.gemm_f32_selected_kernel(M, N, K, K, N, N, P16, Q16, R16)
    # a batch: whole-K MFMA kernels only (no K split, no skinny kernel), sized
    # by the tiles of the whole batch
    for (M, N, K, bt) in [(512, 512, 512, 64), (8, 8192, 8192, 4), (64, 64, 64, 1000),
                          (1000, 999, 777, 3), (256, 256, 256, 100000)]:
        name = sel(M, N, K, K, M * K, N, K * N, N, bt, P16, Q16)
        assert name in names and name.startswith("mfma_") and "_sk_" not in name, name
    # direct-to-LDS kernels need every product 16-byte aligned: strides % 4
    assert "_d6_" in sel(512, 512, 512, 512, 512 * 512, 512, 512 * 512, 512, 64, P16, Q16)
    odd = sel(512, 512, 512, 512, 512 * 512 + 1, 512, 512 * 512, 512, 64, P16, Q16)
    assert odd.startswith("mfma_") and "_d6_" not in odd, odd
    assert sel(4, 4, 4, 4, -1, 4, 16, 4, 2, P16, Q16) == "invalid"
    assert sel(4, 4, 4, 4, 16, 4, 16, 4, -2, P16, Q16) == "invalid"


# ---- deterministic sum (reduce_sum_f32) ------------------------------------------

def test_reduce_sum_argument_errors_before_any_device_call():
    f = binding.reduce_sum_f32
    assert f(-1, P16, R16, 0) == 1
    assert f(10, 0, R16, 0) == 3
    assert f(10, P16, 0, 0) == 3
    assert f(0, 0, 0, 0) == 3            # out is always written
    assert f(10, P16 + 2, R16, 0) == 9
    assert f(10, P16, R16 + 1, 0) == 9
    assert f(10, P16, P16 + 36, 0) == 4  # out is the last element of x
    assert f(10, P16, P16 + 40, 0) != 4  # right after x: not an alias


# ---- fused epilogue (gemm_f32_fused) ---------------------------------------------

def test_fused_argument_errors_before_any_device_call():
    f = binding.gemm_f32_fused
    # unknown activation
    assert f(0, 0, 4, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, 0, 2, 0) == 10
    assert f(0, 0, 4, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, 0, -1, 0) == 10
    # misaligned bias; bias inside C's window
    assert f(0, 0, 4, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, R16 + 0x100002, 1, 0) == 9
    assert f(0, 0, 4, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, R16 + 16, 1, 0) == 4
    # the checks of gemm_f32_ex come first
    assert f(0, 0, -1, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, 0, 7, 0) == 1
    # empty products succeed without a device
    assert f(0, 0, 0, 4, 4, 1.0, P16, 4, Q16, 4, 0.0, R16, 4, 0, 1, 0) == 0


def test_fused_selects_the_extended_kernels():
    """With a bias or an activation the product is not plain: gemm_f32_fused
    runs what gemm_f32_ex runs for alpha, beta other than 1, 0 (the kernel
    choice does not depend on the bias or activation)."""
    names = binding.kernel_names()
    assert any(n.startswith("mfmaex_") for n in names)
    # run_kernel_fused refuses the plain-only kernels for a fused update
    plain = names.index("mfma_64x64x32_w32x32_p5_vec")
    assert binding.gemm_f32_run_kernel_fused(plain, 0, 0, 4, 4, 4, 1.0, P16, 4, Q16, 4, 0.0,
                                             R16, 4, 0, 1, 0) in (5, 8)


def test_extended_skinny_rows_by_width():
    """With an epilogue, A and B as stored: the 16-wave exchange kernel up to
    2048 columns, the 8-wave one above; A stored transposed: its own kernel."""
    sel = binding.gemm_f32_selected_kernel_ex
    assert sel(0, 0, 8, 1024, 8192, 8192, 1024, 1024, 2.0, 1.0, P16, Q16, R16) == \
        "skinnyx_w16_c2_u2_s0_vec"
    assert sel(0, 0, 8, 2049, 8192, 8192, 2049, 2049, 2.0, 1.0, P16, Q16, R16) == \
        "skinnyx_w8_c2_u2_s0_vec"
    assert sel(1, 0, 8, 1024, 8192, 8, 1024, 1024, 2.0, 1.0, P16, Q16, R16) == \
        "skinnyx_w8_c2_u2_s0_tn"


def test_extended_direct_loads_only_under_their_conditions():
    """A transposed operand takes the direct-to-LDS extended kernels only with
    16-byte aligned A and B, lda and ldb multiples of 4, K a multiple of 32,
    M a multiple of 4 when A is transposed and N when B is not; otherwise the
    register-staged kernel of the same row class."""
    sel = binding.gemm_f32_selected_kernel_ex
    for ta, tb in [(0, 1), (1, 0), (1, 1)]:
        lay = f"_{'t' if ta else 'n'}{'t' if tb else 'n'}"
        good = sel(ta, tb, 1024, 1024, 1024, 1024, 1024, 1024, 1.0, 0.0, P16, Q16, R16)
        assert good == "mfmaex_64x64x32_w32x32_d6" + lay, good
        assert sel(ta, tb, 4096, 4096, 4096, 4096, 4096, 4096, 1.0, 0.0, P16, Q16, R16) == \
            "mfmaex_256x256x32_w64x128_d6" + lay
        bad = [
            (1024, 1024, 1040, 1040 if not ta else 1024, 1040 if tb else 1024, P16, Q16),  # K % 32
            (1024, 1024, 1024, 1025, 1025, P16, Q16),                                    # pitches
            (1024, 1024, 1024, 1024, 1024, P16 + 4, Q16),                                # A alignment
        ]
        if ta:
            bad.append((1022, 1024, 1024, 1024, 1024, P16, Q16))                         # M % 4, A^T
        if not tb:
            bad.append((1024, 1022, 1024, 1024, 1024, P16, Q16))                         # N % 4, B
        for M, N, K, lda_, ldb_, pa, pb in bad:
            name = sel(ta, tb, M, N, K, lda_, ldb_, max(N, 1), 1.0, 0.0, pa, pb, R16)
            assert name.startswith("mfmaex_") and "_d6_" not in name, (ta, tb, M, N, K, name)
            assert name.endswith(lay), name
