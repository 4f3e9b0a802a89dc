"""The C-ABI library loads, exports every declared entry point, and validates arguments on
the host without touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import binary_bit_gemm_amd as lb
from binary_bit_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")

OK, INVALID, UNSUPPORTED, ALIGN, HIP, TOO_MANY = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lowbit_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("lowbit_pack", "lowbit_unpack", "lowbit_gemm", "lowbit_gemm_batched"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES), "binding signatures out of date"


def test_version_and_status_strings():
    assert lb.version() == 100
    for s in (OK, INVALID, UNSUPPORTED, ALIGN, HIP, TOO_MANY):
        assert lb.status_string(s) and lb.status_string(s) != "unknown status"
    assert lb.status_string(99) == "unknown status"


A = 0x10000  # a 16-byte-aligned fake address: never dereferenced by the host checks


@pytest.mark.parametrize("args,want", [
    ((A, A, A, A, 64, 256, 256, 64, 2), OK),
    ((A, A, A, A, 64, 256, 256, 64, 3), UNSUPPORTED),        # bits
    ((A, A, A, A, 64, 256, 256, 48, 2), UNSUPPORTED),        # g
    ((A, A, A, A, 64, 256, 256, 16, 1), UNSUPPORTED),
    ((A, A, A, A, 64, 250, 256, 64, 2), INVALID),            # N % 16
    ((A, A, A, A, 64, 256, 200, 64, 2), INVALID),            # K % g
    ((A, A, A, A, -1, 256, 256, 64, 2), INVALID),
    ((A, A, A, A, 64, 256, 1 << 31, 64, 2), INVALID),
    ((0, A, A, A, 64, 256, 256, 64, 2), INVALID),            # null X
    ((A, 0, A, A, 64, 256, 256, 64, 2), INVALID),
    ((A, A, 0, A, 64, 256, 256, 64, 2), INVALID),
    ((A, A, A, 0, 64, 256, 256, 64, 2), INVALID),
    ((A + 8, A, A, A, 64, 256, 256, 64, 2), ALIGN),
    ((A, A + 4, A, A, 64, 256, 256, 64, 2), ALIGN),
    ((A, A, A + 2, A, 64, 256, 256, 64, 2), ALIGN),
    ((A, A, A, A + 2, 64, 256, 256, 64, 2), ALIGN),
    ((0, 0, 0, 0, 0, 256, 256, 64, 2), OK),                   # M == 0: nothing to do
    ((0, 0, 0, A, 64, 256, 0, 64, 2), OK),                    # K == 0: Y = 0, no inputs read
    ((A, A, A, A, 64, 256, 256, 128, 1), OK),
    ((A, A, A, A, 64, 256, 256, 32, 1), OK),
    ((A, A, A, A, 64, 256, 1 << 22, 64, 2), OK),               # size limits of the kernels' addressing
    ((A, A, A, A, 64, 256, (1 << 22) + 64, 64, 2), UNSUPPORTED),
    ((A, A, A, A, 64, (1 << 20) - 16, 1 << 14, 64, 2), OK),    # packed weights 4 GiB - 64 KiB ...
    ((A, A, A, A, 64, 1 << 20, 1 << 14, 64, 2), UNSUPPORTED),  # ... and exactly 4 GiB
    ((A, A, A, A, 64, 1 << 21, 1 << 15, 64, 1), UNSUPPORTED),  # binary: 8 GiB
    ((A, A, A, A, 1 << 30, 1 << 7, 256, 64, 2), OK),           # M*N = 2^37
    ((A, A, A, A, 1 << 30, 1 << 8, 256, 64, 2), UNSUPPORTED),
])
def test_check_gemm_args(args, want):
    assert lb.check_gemm_args(*args) == want


def test_gemm_rejects_before_touching_the_device():
    L = _lib.lib()
    st = L.lowbit_gemm(A, A, A, A, 64, 250, 256, 64, 2, None)
    assert st == INVALID
    st = L.lowbit_pack(A, A, 16, 24, 2, None, None)  # K not a multiple of 16
    assert st == INVALID
    st = L.lowbit_unpack(A, A, 16, 32, 5, None)
    assert st == UNSUPPORTED
    assert L.lowbit_pack(A, A, 1 << 21, 1 << 20, 2, None, None) == UNSUPPORTED  # 2^41 codes
    assert L.lowbit_gemm(A, A, A, A, 64, 1 << 20, 1 << 14, 64, 2, None) == UNSUPPORTED  # 4 GiB of words
    probs = (lb.Problem * 2)()
    probs[0] = lb.Problem(A, A, A, A, 64, 256, 256, 64, 2)
    probs[1] = lb.Problem(A, A, A, A, 64, 256, 256, 64, 7)
    assert L.lowbit_gemm_batched(probs, 2, None) == UNSUPPORTED
    assert L.lowbit_gemm_batched(probs, lb.MAX_BATCH + 1, None) == TOO_MANY
    assert L.lowbit_gemm_batched(None, 3, None) == INVALID
    assert L.lowbit_gemm_batched(None, 0, None) == OK


def test_swiglu_rejects_before_touching_the_device():
    """lowbit_gemm_swiglu validates as lowbit_gemm with 2N weight rows, and takes g = 64 / 128 only."""
    L = _lib.lib()
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, 250, 256, 64, 2, None) == INVALID      # N % 16
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, 256, 200, 64, 2, None) == INVALID      # K % g
    assert L.lowbit_gemm_swiglu(0, A, A, A, 64, 256, 256, 64, 2, None) == INVALID      # null X
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, -16, 256, 64, 2, None) == INVALID
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, 256, 256, 32, 2, None) == UNSUPPORTED  # g = 32
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, 256, 256, 64, 3, None) == UNSUPPORTED  # bits
    assert L.lowbit_gemm_swiglu(A + 8, A, A, A, 64, 256, 256, 64, 2, None) == ALIGN
    # 2N rows of packed words: 2 x (2^19 rows x 4 KiB) = 4 GiB
    assert L.lowbit_gemm_swiglu(A, A, A, A, 64, 1 << 19, 1 << 14, 64, 2, None) == UNSUPPORTED
    assert L.lowbit_gemm_swiglu(0, 0, 0, 0, 0, 256, 256, 64, 2, None) == OK            # M == 0


def test_residual_rejects_before_touching_the_device():
    """lowbit_gemm_residual validates as lowbit_gemm, plus its residual and gate pointers."""
    L = _lib.lib()
    assert L.lowbit_gemm_residual(A, A, A, A, A, A, 64, 250, 256, 64, 2, None) == INVALID      # N % 16
    assert L.lowbit_gemm_residual(A, A, A, 0, A, A, 64, 256, 256, 64, 2, None) == INVALID      # null R
    assert L.lowbit_gemm_residual(A, A, A, A, 0, A, 64, 256, 256, 64, 2, None) == INVALID      # null gate
    assert L.lowbit_gemm_residual(A, A, A, A + 2, A, A, 64, 256, 256, 64, 2, None) == ALIGN
    assert L.lowbit_gemm_residual(A, A, A, A, A + 2, A, 64, 256, 256, 64, 2, None) == ALIGN
    assert L.lowbit_gemm_residual(A, A, A, A, A, A, 64, 256, 256, 32, 2, None) == UNSUPPORTED  # g = 32
    assert L.lowbit_gemm_residual(0, 0, 0, 0, 0, 0, 0, 256, 256, 64, 2, None) == OK            # M == 0


def test_import_rejects_before_touching_the_device():
    """lowbit_import_ternary validates layout, zero point, shape, size and alignment first."""
    L = _lib.lib()
    GL, MLX = lb.LAYOUT_GEMLITE_U8T, lb.LAYOUT_MLX_U32
    assert (GL, MLX) == (1, 2)
    assert L.lowbit_import_ternary(A, 3, 1, A, 64, 256, None, None) == INVALID                  # layout
    assert L.lowbit_import_ternary(A, GL, 4, A, 64, 256, None, None) == INVALID                 # zero
    assert L.lowbit_import_ternary(A, GL, -1, A, 64, 256, None, None) == INVALID
    assert L.lowbit_import_ternary(A, GL, 1, A, 40, 256, None, None) == INVALID                 # N % 16
    assert L.lowbit_import_ternary(A, MLX, 1, A, 64, 264, None, None) == INVALID                # K % 16
    assert L.lowbit_import_ternary(A, GL, 1, A, 16, (1 << 22) + 16, None, None) == UNSUPPORTED  # K > 2^22
    assert L.lowbit_import_ternary(0, GL, 1, A, 64, 256, None, None) == INVALID                 # null src
    assert L.lowbit_import_ternary(A + 4, GL, 1, A, 64, 256, None, None) == ALIGN
    assert L.lowbit_import_ternary(A, MLX, 1, A + 8, 64, 256, None, None) == ALIGN
    assert L.lowbit_import_ternary(0, GL, 1, 0, 0, 256, None, None) == OK                       # empty
    assert L.lowbit_import_binary_gemlite(A, A, 40, 256, None) == INVALID                        # N % 16
    assert L.lowbit_import_binary_gemlite(A, A, 64, 48, None) == INVALID                         # K % 32
    assert L.lowbit_import_binary_gemlite(A + 4, A, 64, 256, None) == ALIGN
    assert L.lowbit_import_binary_gemlite(A, A, 16, (1 << 22) + 32, None) == UNSUPPORTED
    assert L.lowbit_import_binary_gemlite(0, 0, 0, 256, None) == OK


def test_int4_arguments_and_kernel():
    """4-bit codes: g = 64 / 128 on the 16x16-block tile kernel at every M (forced variants of
    other kernels included); g = 32 and other bit widths are refused."""
    L = _lib.lib()
    assert L.lowbit_check_gemm_args(A, A, A, A, 512, 2560, 9728, 64, 4) == OK
    assert L.lowbit_check_gemm_args(A, A, A, A, 512, 2560, 9728, 128, 4) == OK
    assert L.lowbit_check_gemm_args(A, A, A, A, 512, 2560, 9728, 32, 4) == UNSUPPORTED
    assert L.lowbit_check_gemm_args(A, A, A, A, 512, 2560, 9728, 64, 3) == UNSUPPORTED
    assert L.lowbit_pack(A, A, 16, 12, 4, None, None) == INVALID          # K % 8
    assert L.lowbit_pack(A, A, 16, 24, 3, None, None) == UNSUPPORTED
    tile16 = {"tile288x192", "tile256x192", "tile96x192", "tile96x192k2", "tile64x128k2"}
    for M, N, K in ((1, 16, 64), (16, 3072, 2560), (512, 19456, 2560), (512, 2560, 9728), (4608, 3072, 3072)):
        assert lb.variant(M, N, K, 64, 4) in tile16, (M, N, K)


def test_int4_forced_variants_stay_on_the_tile16_kernel(monkeypatch):
    for v in ("skinny", "resident", "tile64", "tile256w"):
        monkeypatch.setenv("LOWBIT_VARIANT", v)
        assert lb.variant(16, 3072, 2560, 64, 4) in {"tile288x192", "tile256x192", "tile96x192", "tile96x192k2",
                                                     "tile64x128k2"}, v


def test_variant_choice():
    """Tile choice: fewest rounds of tiles over 256 compute units, weighted by tile work.
    4608 x 3072 is 216 tiles of 256 x 256 (40 units idle) but exactly 256 of 288 x 192."""
    assert lb.variant(4608, 3072, 3072, 64, 2) == "tile288x192"
    assert lb.variant(4608, 18432, 3072, 64, 2) == "tile288x192"
    assert lb.variant(4608, 3072, 12288, 128, 2) == "tile288x192"
    # the 16x16-block kernel takes g = 64 / 128; for binary codes it does less work per unit
    # time than 256 x 256 by more than the idle units cost, so binary stays on 256 x 256
    assert lb.variant(4608, 3072, 3072, 64, 1) == "tile256x256"
    assert lb.variant(4608, 3072, 12288, 128, 1) == "tile256x256"
    assert lb.variant(4608, 3072, 3072, 32, 2) == "tile256x256"
    assert lb.variant(4608, 3072, 3072, 32, 1) == "tile256x256"
    # M = 1536: 96 x 192 tiles fill the chip at N = 3072 (256 tiles, one round), with K split
    # between two groups of waves where the step count is even; 256 x 256 wins above
    assert lb.variant(1536, 3072, 3072, 64, 2) == "tile96x192k2"
    assert lb.variant(1536, 3072, 9216, 64, 1) == "tile96x192k2"
    assert lb.variant(1536, 3072, 3136, 64, 2) == "tile96x192"  # 49 steps
    assert lb.variant(1536, 9216, 3072, 64, 2) == "tile256x256"
    # M = 4096 (the image stream's linears as single calls): 256 x 192 tiles make whole rounds at
    # N = 3072 and 9216 where 288 x 192 needs a 22%-full last row of tiles; at N = 18432 256 x 256
    # still wins; M = 4608 stays on 288 x 192 (256 x 192 would need 18 rows: 1.125 rounds)
    assert lb.variant(4096, 3072, 3072, 64, 2) == "tile256x192"
    assert lb.variant(4096, 9216, 3072, 64, 2) == "tile256x192"
    assert lb.variant(4096, 3072, 9216, 128, 1) == "tile256x192"
    assert lb.variant(4096, 18432, 3072, 64, 2) == "tile256x256"
    assert lb.variant(512, 19456, 2560, 64, 4) == "tile256x192"
    assert not lb.variant(1536, 3072, 3072, 32, 2).startswith("tile96")  # g = 32: 32x32-block kernel only
    assert lb.variant(64, 256, 256, 64, 2).startswith("tile")


def test_skinny_variant_choice():
    """The skinny kernel takes M <= 32 (ternary) / M <= 16 (binary) for g = 32 / 64 / 128 when
    K is a whole number of 64-byte row steps (a 16-byte chunk larger than a group -- 64
    ternary or 128 binary codes -- runs each of its MFMAs once per group)."""
    assert lb.variant(16, 3072, 3072, 64, 2) == "skinny"
    assert lb.variant(1, 3072, 3072, 128, 2) == "skinny"
    assert lb.variant(32, 3072, 12288, 64, 2) == "skinny"
    assert lb.variant(33, 3072, 3072, 64, 2) == "tile64x256"
    assert lb.variant(16, 3072, 3072, 32, 2) == "skinny"         # chunk of 64 over two groups
    assert lb.variant(16, 3072, 320, 64, 2) == "tile64x256"      # K % 256 != 0
    assert lb.variant(16, 3072, 3072, 128, 1) == "skinny"
    assert lb.variant(16, 3072, 3072, 64, 1) == "skinny"         # binary chunk over two groups
    assert lb.variant(16, 3072, 3072, 32, 1) == "skinny"         # ... or four
    assert lb.variant(16, 3072, 2816, 128, 1) == "tile64x256"    # K % 512 != 0
    assert lb.variant(17, 3072, 3072, 128, 1) == "tile64x256"


def test_resident_variant_and_workspace_size():
    """The resident kernel takes M <= 16 ternary g = 64 / 128 problems; without a workspace
    from 512 column blocks up (N = 27648), whole K.  With a workspace, problems whose K is too
    long for the activations to stay in LDS split K across workgroups: arrival counters +
    fp32 partials of 16 x 16 outputs per column block and K range."""
    assert lb.variant(16, 27648, 3072, 64, 2) == "resident"
    assert lb.variant(16, 27648, 3072, 128, 2) == "resident"
    assert lb.variant(16, 9216, 3072, 64, 2) == "resident"
    assert lb.variant(16, 3072, 3072, 64, 2) == "skinny"
    assert lb.variant(17, 27648, 3072, 64, 2) == "skinny"
    assert lb.variant(16, 27648, 3072, 128, 1) == "skinny"
    assert lb.workspace_size(16, 27648, 3072, 64, 2) == 0     # whole K
    n = lb.workspace_size(16, 3072, 12288, 64, 2)
    assert n > 0 and n % 256 == 0
    assert n >= 2 * 3072 * 16 * 4                             # at least two K ranges of partials
    assert lb.workspace_size(16, 3072, 3072, 64, 2) == 0      # the whole K fits: no split
    assert lb.workspace_size(16, 512, 6144, 128, 2) > 0       # 24 steps of activations do not
    assert lb.workspace_size(16, 3072, 12288, 32, 2) == 0     # group smaller than a piece
    assert lb.workspace_size(32, 3072, 12288, 64, 2) == 0     # two row blocks
    assert lb.workspace_size(16, 3072, 12288, 64, 1) == 0     # binary
    assert lb.workspace_size(16, 3072, 12200, 64, 2) == 0     # K % g != 0: invalid
    assert lb.workspace_size(16, 3000, 12288, 64, 2) == 0     # N % 16 != 0: invalid
    L = lb.lib()
    probs = (lb.Problem * 2)()
    probs[0] = lb.Problem(A, A, A, A, 16, 3072, 9216, 64, 2)
    probs[1] = lb.Problem(A, A, A, A, 16, 3072, 9216, 64, 2)
    assert L.lowbit_batched_workspace_size(probs, 2) > 0     # K-heavy pair: split
    probs[0] = lb.Problem(A, A, A, A, 16, 18432, 3072, 64, 2)
    probs[1] = lb.Problem(A, A, A, A, 16, 18432, 3072, 64, 2)
    assert L.lowbit_batched_workspace_size(probs, 2) == 0    # wide pair: whole K


def test_gemm_ex_validates_before_the_device():
    L = lb.lib()
    A = 256
    assert L.lowbit_gemm_ex(A, A, A, A, 16, 3072, 3072, 64, 2, A + 8, 1 << 20, None) == ALIGN
    assert L.lowbit_gemm_ex(None, A, A, A, 16, 3072, 3072, 64, 2, A, 1 << 20, None) == INVALID
    assert L.lowbit_gemm_ex(A, A, A, A, 16, 3072, 3072, 64, 3, A, 1 << 20, None) == UNSUPPORTED
    assert L.lowbit_gemm_ex(A, A, A, A, 0, 3072, 3072, 64, 2, None, 0, None) == OK


SCRATCH = 6


def test_streamk_workspace_size(monkeypatch):
    # stream-K (LOWBIT_VARIANT=tile256sk): the counters plus two 256 KiB partial tiles per workgroup,
    # one workgroup per compute unit (fewer where the problem has fewer (tile, step) units)
    sk = 4096 + 2 * 256 * 256 * 256 * 4
    assert lb.workspace_size(1536, 18432, 3072, 64, 2) == 0      # the automatic choice: no split
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256sk")
    assert lb.workspace_size(1536, 18432, 3072, 64, 2) == sk
    assert lb.workspace_size(4608, 9216, 3072, 128, 1) == sk
    assert lb.workspace_size(256, 256, 640, 64, 2) == 4096 + 2 * 10 * 256 * 256 * 4   # 10 units
    assert lb.workspace_size(1536, 18432, 3072, 64, 4) == 0      # 4-bit codes: the 16x16-block tile
    assert lb.workspace_size(65536, 65536, 4096, 64, 2) > 0      # 2^22 units
    assert lb.workspace_size(65536, 65536, 8192, 64, 2) == 0     # 2^23 units x 256 workgroups = 2^31
    L = lb.lib()
    A = 256
    # forced variants run as lowbit_gemm in the allocation-free entry point: no scratch error
    assert L.lowbit_gemm_noalloc(A, A, A, A + 8, 1536, 18432, 3072, 64, 2, None) == ALIGN


def test_noalloc_validates_before_the_device(monkeypatch):
    L = lb.lib()
    A = 256
    assert lb.status_string(SCRATCH) and lb.status_string(SCRATCH) != "unknown status"
    assert L.lowbit_gemm_noalloc(None, A, A, A, 16, 3072, 3072, 64, 2, None) == INVALID
    assert L.lowbit_gemm_noalloc(A, A, A, A + 8, 16, 3072, 3072, 64, 2, None) == ALIGN
    assert L.lowbit_gemm_noalloc(A, A, A, A, 16, 3072, 3072, 64, 3, None) == UNSUPPORTED
    assert L.lowbit_gemm_noalloc(A, A, A, A, 0, 3072, 3072, 64, 2, None) == OK
    # every automatic split plan fits the static scratch ...
    for (M, N, K) in ((16, 3072, 12288), (16, 18432, 9216), (1, 4096, 65536), (8, 18432, 12288)):
        assert 0 < lb.workspace_size(M, N, K, 64, 2) <= lb.NOALLOC_SCRATCH_BYTES, (M, N, K)
    # ... a forced plan that needs more is refused before anything touches a device
    monkeypatch.setenv("LOWBIT_RESIDENT_PLAN", "1,16")
    assert lb.workspace_size(16, 16384, 16384, 64, 2) > lb.NOALLOC_SCRATCH_BYTES
    assert L.lowbit_gemm_noalloc(A, A, A, A, 16, 16384, 16384, 64, 2, None) == SCRATCH


def test_affine_entry_points_validate_before_the_device():
    L = lb.lib()
    A = 256
    # lowbit_pack_u4: K % 8, alignment, nulls
    assert L.lowbit_pack_u4(A, A, 16, 12, None, None) == INVALID
    assert L.lowbit_pack_u4(A + 4, A, 16, 64, None, None) == ALIGN
    assert L.lowbit_pack_u4(None, A, 16, 64, None, None) == INVALID
    assert L.lowbit_pack_u4(None, None, 0, 64, None, None) == OK
    # lowbit_gemm_affine: 4-bit rules (g = 32 unsupported), the bias pointer checked like the others
    assert L.lowbit_gemm_affine(A, A, A, A, A, 16, 256, 256, 32, None) == UNSUPPORTED
    assert L.lowbit_gemm_affine(A, A, A, None, A, 16, 256, 256, 64, None) == INVALID
    assert L.lowbit_gemm_affine(A, A, A, A + 2, A, 16, 256, 256, 64, None) == ALIGN
    assert L.lowbit_gemm_affine(A, A, A, A, A, 16, 250, 256, 64, None) == INVALID
    assert L.lowbit_gemm_affine(A, A, A, A, A, 0, 256, 256, 64, None) == OK
