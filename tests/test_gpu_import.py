"""GPU parity of the importers (lowbit_import_ternary: GemLite transposed uint8 and MLX uint32
rows; lowbit_import_binary_gemlite: GemLite's transposed 1-bit bytes) against the oracle, through
the C-ABI: bit-exact words and the same count of invalid levels."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, host_words, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _gemlite(src_u8, N, K, zero):
    got, bad = lb.import_gemlite(torch().from_numpy(src_u8).cuda(), N, K, zero)
    return host_words(got), bad


def _mlx(src_u32, N, K, zero):
    got, bad = lb.import_mlx(torch().from_numpy(src_u32.view(np.int32)).cuda(), N, K, zero)
    return host_words(got), bad


def _expect(decoded):
    codes, bad = decoded
    words, _ = oracle.pack(codes, 2)
    return words, bad


# (N, K): one tile, ragged tiles in both directions (N % 64 == 16, K / 16 == 65 words), the
# smallest shape, a square weight (the orientation the buffer's shape cannot tell), and the
# MMDiT's 3072 -> 9216 linear
SHAPES = [(64, 256), (208, 1040), (16, 16), (3072, 3072), (9216, 3072), (1008, 4352)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("zero", [1, 0, 2, 3])
def test_import_random_levels(N, K, zero):
    """Uniform random levels 0..3 (so some fields are no ternary code at every zero point)."""
    rng = np.random.default_rng(N * 7 + K + zero)
    gl = rng.integers(0, 256, size=(K // 4, N), dtype=np.uint8)
    got, bad = _gemlite(gl, N, K, zero)
    want, want_bad = _expect(oracle.gemlite_u8t_decode(gl, N, K, zero))
    assert bad == want_bad and np.array_equal(got, want), f"gemlite {N}x{K} zero {zero}"
    ml = rng.integers(0, 1 << 32, size=(N, K // 16), dtype=np.uint32)
    got, bad = _mlx(ml, N, K, zero)
    want, want_bad = _expect(oracle.mlx_u32_decode(ml, N, K, zero))
    assert bad == want_bad and np.array_equal(got, want), f"mlx {N}x{K} zero {zero}"


@pytest.mark.parametrize("N,K", [(3072, 3072), (208, 1040)])
def test_import_gives_the_packed_weight(N, K):
    """A ternary weight of the workload's code mix, exported to either layout by the oracle and
    imported on the GPU, equals lowbit_pack of its codes word for word, with nothing invalid."""
    codes = W.gen_codes(np.random.default_rng(K + N), N, K, 2)
    packed, bad = lb.pack(dev_codes(codes), 2)
    assert bad == 0
    packed = host_words(packed)
    got, bad = _gemlite(oracle.gemlite_u8t_encode(codes), N, K, 1)
    assert bad == 0 and np.array_equal(got, packed)
    got, bad = _mlx(oracle.mlx_u32_encode(codes), N, K, 1)
    assert bad == 0 and np.array_equal(got, packed)


def test_imported_weight_runs_the_gemm():
    """An imported GemLite weight gives the oracle's Y through lowbit_gemm."""
    M, N, K, g = 96, 3072, 3072, 64
    p = W.Problem("import", M, N, K, 2, g, 92, 5)
    inp = W.make_inputs(p, 0)
    t = torch()
    words, bad = lb.import_gemlite(t.from_numpy(oracle.gemlite_u8t_encode(inp.codes)).cuda(), N, K)
    assert bad == 0
    y = host_bits(lb.gemm(dev_x(inp.x), words, dev_scales(inp.scales), g, 2))
    r = oracle.check_tolerance(y, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
    assert r["ok"], r


def test_import_shape_is_checked_not_guessed():
    """The binding takes N and K from the caller: a square weight's (K/4, N) buffer is refused
    for a shape that would read it in the direct orientation."""
    t = torch()
    src = t.zeros((768, 3072), dtype=t.uint8, device="cuda")     # 3072 x 3072 weight
    with pytest.raises(ValueError):
        lb.import_gemlite(src, 768, 12288)                         # the direct reading's shape
    words, bad = lb.import_gemlite(src, 3072, 3072, zero=0)        # level 0 at zero 0: code 0
    assert bad == 0 and words.shape == (3072, 192) and not t.any(words).item()


@pytest.mark.parametrize("N,K", [(64, 256), (208, 1056), (16, 32), (3072, 3072), (9216, 3072)])
def test_import_gemlite_binary(N, K):
    """GemLite 1-bit bytes [K/8, N] -> binary words, bit-exact against the oracle's decode and
    pack (random bytes: every pattern is a code), on one tile, ragged tiles (N % 64 == 16, 33
    words a row), the smallest shape, a square weight and the 3072 -> 9216 linear."""
    rng = np.random.default_rng(N + 3 * K)
    src = rng.integers(0, 256, size=(K // 8, N), dtype=np.uint8)
    got = host_words(lb.import_gemlite_binary(torch().from_numpy(src).cuda(), N, K))
    want, bad = oracle.pack(oracle.gemlite_binary_decode(src, N, K), 1)
    assert bad == 0 and np.array_equal(got, want)


def test_imported_binary_weight_runs_the_gemm():
    """The binary card's format end to end: GemLite 1-bit bytes, g = 128, through lowbit_gemm."""
    M, N, K, g = 64, 3072, 3072, 128
    inp = W.make_inputs(W.Problem("import_b", M, N, K, 1, g, 92, 6), 0)
    words = lb.import_gemlite_binary(torch().from_numpy(oracle.gemlite_binary_encode(inp.codes)).cuda(), N, K)
    y = host_bits(lb.gemm(dev_x(inp.x), words, dev_scales(inp.scales), g, 1))
    r = oracle.check_tolerance(y, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
    assert r["ok"], r
