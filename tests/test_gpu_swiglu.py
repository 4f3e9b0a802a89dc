"""GPU parity of the fused SwiGLU entry point (lowbit_gemm_swiglu: Y = silu(X . Wg^T) * (X . Wu^T)
with the weights holding gate rows then up rows) against the oracle, through the C-ABI."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _inputs(M, N, K, g, bits, seed=0):
    """Inputs of a [gate | up] weight of 2N rows."""
    p = W.Problem("swiglu", M, 2 * N, K, bits, g, 90, (M * 5 + N * 3 + K + g + bits) % 100000)
    return W.make_inputs(p, seed)


def _run(inp, g, bits):
    x = dev_x(inp.x)
    words, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    s = dev_scales(inp.scales)
    y = lb.gemm_swiglu(x, words, s, g, bits)
    torch().cuda.synchronize()
    return host_bits(y), (x, words, s)


def _check(y_bits, inp, g, what, cols=None):
    N = inp.codes.shape[0] // 2
    if cols is None:
        ref = oracle.swiglu_ref_f64(inp.x, inp.codes, inp.scales, g)
        got = y_bits
    else:  # output column n depends on weight rows n and N + n only
        rows = np.concatenate([cols, N + cols])
        ref = oracle.swiglu_ref_f64(inp.x, inp.codes[rows], inp.scales[rows], g)
        got = y_bits[:, cols]
    r = oracle.check_tolerance(got, ref)
    assert r["ok"], f"{what}: {r}"
    # logic-error alarm: well above the bf16 output rounding floor, which for a few outputs can
    # itself exceed REL_ALARM (16 outputs: 2.5e-3 measured)
    floor = oracle.check_tolerance(oracle.f64_to_bf16_bits_rne(ref), ref)["rel_frob"]
    assert r["rel_frob"] <= max(REL_ALARM, 1.5 * floor), f"{what}: rel_frob {r['rel_frob']} (floor {floor})"


# (M, N, K, g, bits): several M and N tiles with ragged edges (N % 96 != 0 leaves a partly
# filled last tile whose gate and up rows past N are re-read and not stored), one K step,
# K long enough to cross several weight and scale blocks, g = 128 and binary codes
SHAPES = [(300, 400, 1280, 64, 2), (577, 96, 3072, 128, 2), (16, 208, 512, 64, 1), (289, 1008, 2304, 128, 1),
          (1, 16, 64, 64, 2), (96, 112, 8448, 64, 2)]


@pytest.mark.parametrize("M,N,K,g,bits", SHAPES)
def test_swiglu_parity(M, N, K, g, bits):
    inp = _inputs(M, N, K, g, bits)
    y, _ = _run(inp, g, bits)
    _check(y, inp, g, f"swiglu {M}x{N}x{K} g{g} b{bits}")


# skinny M (ternary, K % 256 == 0): the resident kernel's SwiGLU mode where a whole-K plan fits
# (workgroups of gate blocks and the matching up blocks), the tile kernel otherwise (K = 12288
# at M = 16 does not fit one workgroup's LDS)
SKINNY = [(16, 9216, 3072, 64), (5, 400, 1280, 128), (16, 1008, 4352, 64), (1, 16, 256, 64), (16, 3072, 12288, 64),
          (11, 3072, 9216, 128)]


@pytest.mark.parametrize("M,N,K,g", SKINNY)
def test_swiglu_skinny_parity(M, N, K, g):
    inp = _inputs(M, N, K, g, 2, seed=7)
    y, _ = _run(inp, g, 2)
    _check(y, inp, g, f"swiglu skinny {M}x{N}x{K} g{g}")


def test_swiglu_mlp_in_full_size_sampled():
    """The MMDiT's MLP-in at 1024^2 (M = 4608, 2 x 9216 outputs, K = 3072, ternary g = 64), in the
    launch configuration bench.py times; sampled output columns against the oracle."""
    M, N, K, g, bits = 4608, 9216, 3072, 64, 2
    inp = _inputs(M, N, K, g, bits, seed=2)
    y, _ = _run(inp, g, bits)
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 96, replace=False)]))
    _check(y, inp, g, "swiglu 4608x9216x3072 (sampled)", cols=cols)


def test_swiglu_matches_its_two_gemms():
    """The fused result is silu(gate) * up of the two plain GEMMs up to the bf16 rounding of those
    GEMMs' outputs (the fused path rounds once), and two calls are bitwise equal."""
    t = torch()
    M, N, K, g, bits = 300, 384, 1024, 64, 2
    inp = _inputs(M, N, K, g, bits, seed=5)
    y, (x, words, s) = _run(inp, g, bits)
    y2 = host_bits(lb.gemm_swiglu(x, words, s, g, bits))
    assert np.array_equal(y, y2)
    gt = lb.gemm(x, words[:N].contiguous(), s[:N].contiguous(), g, bits).double()
    up = lb.gemm(x, words[N:].contiguous(), s[N:].contiguous(), g, bits).double()
    comp = (gt / (1.0 + t.exp(-gt)) * up).cpu().numpy()
    r = oracle.check_tolerance(y, comp, rel_frob_tol=5e-3, elem_tol=1e-2)
    assert r["ok"], r


def test_swiglu_k0_and_empty():
    t = torch()
    x0 = t.zeros((5, 0), dtype=t.bfloat16, device="cuda")
    w0 = t.zeros((64, 0), dtype=t.int32, device="cuda")
    s0 = t.zeros((64, 0), dtype=t.float16, device="cuda")
    y = t.full((5, 32), 7.0, dtype=t.bfloat16, device="cuda")
    lb.gemm_swiglu(x0, w0, s0, 64, 2, out=y)
    assert not y.float().abs().sum().item()
    x = t.zeros((0, 64), dtype=t.bfloat16, device="cuda")
    w = t.zeros((32, 4), dtype=t.int32, device="cuda")
    s = t.ones((32, 1), dtype=t.float16, device="cuda")
    assert lb.gemm_swiglu(x, w, s, 64, 2).shape == (0, 16)


def test_swiglu_rejects_g32_and_odd_rows():
    t = torch()
    x = t.zeros((4, 64), dtype=t.bfloat16, device="cuda")
    w = t.zeros((32, 4), dtype=t.int32, device="cuda")
    s = t.ones((32, 2), dtype=t.float16, device="cuda")
    with pytest.raises(lb.LowbitError):
        lb.gemm_swiglu(x, w, s, 32, 2)
    with pytest.raises(ValueError):
        lb.gemm_swiglu(x, w[:31], s[:31, :1], 64, 2)


def test_swiglu_on_the_fused_single_stream_linear():
    """The single-stream 3072 -> 27648 linear holds [QKV 9216 | gate 9216 | up 9216] rows; its
    MLP part takes the fused SwiGLU and its QKV part the plain GEMM, as two calls on row slices of
    the one packed weight (offset pointers into the same buffers, no copy); sampled columns
    against the oracle."""
    t = torch()
    M, K, g, bits, H = 96, 3072, 64, 2, 9216
    p = W.Problem("single_fused", M, 3 * H, K, bits, g, 90, 77)
    inp = W.make_inputs(p, 0)
    x = dev_x(inp.x)
    words, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    s = dev_scales(inp.scales)
    qkv = host_bits(lb.gemm(x, words[:H], s[:H], g, bits))
    mlp = host_bits(lb.gemm_swiglu(x, words[H:], s[H:], g, bits))
    t.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(8), np.arange(H - 8, H), np.random.default_rng(4).choice(H, 48, replace=False)]))
    r = oracle.check_tolerance(qkv[:, cols], oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], g))
    assert r["ok"], r
    rows = np.concatenate([H + cols, 2 * H + cols])
    ref = oracle.swiglu_ref_f64(inp.x, inp.codes[rows], inp.scales[rows], g)
    r = oracle.check_tolerance(mlp[:, cols], ref)
    assert r["ok"], r
