"""GPU parity of the skinny-M kernel (M <= 32) against the oracle, through the C-ABI.

Covers every compiled configuration (ternary g = 64 / 128 with one and two 16-row blocks,
binary g = 128; stripes of 1, 2 and 4 column blocks), wave step ranges that are empty,
uneven or odd, rows past M, and the bit-exact identities on this path."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import run_gemm, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _inputs(M, N, K, g, bits, seed=0, cid=40):
    p = W.Problem("skinny", M, N, K, bits, g, cid, (M * 7 + N * 3 + K + g + bits) % 100000)
    return W.make_inputs(p, seed)


def _check(M, N, K, g, bits, seed=0, what=""):
    assert lb.variant(M, N, K, g, bits) == "skinny", (M, N, K, g, bits)
    inp = _inputs(M, N, K, g, bits, seed)
    y, _ = run_gemm(inp, g, bits)
    r = oracle.check_tolerance(y, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
    assert r["ok"], f"{what} {M}x{N}x{K} g{g} b{bits}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']}"


def _is_zero(bits):
    return (bits & 0x7FFF) == 0


# (bits, g, K): K = 5 row steps, so the four waves get 1, 1, 1 and 2 steps
_FORMATS = [(2, 64, 1280), (2, 128, 1280), (1, 128, 2560), (1, 64, 2560), (2, 32, 1280), (1, 32, 2560)]


@pytest.mark.parametrize("bits,g,K", _FORMATS)
@pytest.mark.parametrize("ncb", [1, 2, 4])
def test_every_stripe_width(bits, g, K, ncb, monkeypatch):
    monkeypatch.setenv("LOWBIT_SKINNY_NCB", str(ncb))
    _check(16, 2048, K, g, bits, what=f"ncb={ncb}")


@pytest.mark.parametrize("M", [1, 5, 16, 17, 31, 32])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_rows(M, g):
    # 65 column blocks: only one-block stripes divide N
    _check(M, 1040, 768, g, 2, seed=1, what="rows")


@pytest.mark.parametrize("M", [1, 9, 16])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_rows_binary(M, g):
    _check(M, 1040, 1536, g, 1, seed=2, what=f"rows binary g{g}")


@pytest.mark.parametrize("K", [256, 512, 768, 2048, 9216])
def test_step_counts(K):
    # 1 step (three idle waves), 2, 3, 8 and 36 steps
    _check(16, 512, K, 64, 2, seed=3, what="steps")


@pytest.mark.parametrize("bits,g", [(2, 64), (2, 128), (1, 128), (1, 64), (2, 32), (1, 32)])
def test_one_hot_bit_exact(bits, g):
    M, N, K = 16, 64, 1024
    x = W.gen_x(W.rng_for(4, 41, 0), M, K)
    s = W.gen_scales(W.rng_for(4, 41, 1), N, K, g)
    xf = oracle.bf16_bits_to_f64(x)
    for (n0, k0, c0) in ((0, 0, 1), (15, 63, -1), (16, 64, 1), (63, 1023, -1), (37, 517, 1)):
        if bits == 2:
            c = np.zeros((N, K), dtype=np.int8)
        else:  # binary has no zero code: alternating signs, one flipped at (n0, k0)
            c = np.ones((N, K), dtype=np.int8)
            c[:, 1::2] = -1
        c[n0, k0] = c0
        inp = W.Inputs(x, c, s)
        y, _ = run_gemm(inp, g, bits)
        if bits == 2:
            want = oracle.f64_to_bf16_bits_rne(c0 * float(s[n0, k0 // g]) * xf[:, k0])
            col = y[:, n0]
            same = (col == want) | (_is_zero(col) & _is_zero(want))
            assert same.all(), (n0, k0, np.nonzero(~same)[0][:5])
            assert np.all(_is_zero(np.delete(y, n0, axis=1)))
        else:
            ref = oracle.gemm_ref_f64(x, c, s, g)
            assert oracle.check_tolerance(y, ref)["ok"]


def test_zero_codes_scales_and_unused_field():
    M, N, K, g = 16, 256, 1024, 64
    inp = _inputs(M, N, K, g, 2, seed=5)
    y0, _ = run_gemm(W.Inputs(inp.x, np.zeros_like(inp.codes), inp.scales), g, 2)
    assert np.all(_is_zero(y0))
    s = inp.scales.copy()
    s[:, 3] = 0
    c = inp.codes.copy()
    c[:, 3 * g:4 * g] = 0
    ya, _ = run_gemm(W.Inputs(inp.x, inp.codes, s), g, 2)
    yc, _ = run_gemm(W.Inputs(inp.x, c, inp.scales), g, 2)
    assert ((ya == yc) | (_is_zero(ya) & _is_zero(yc))).all()
    # words of all-ones fields (the unused ternary pattern 11) decode to 0
    t = torch()
    from tests.gpu_helpers import dev_scales, dev_x
    words = t.full((N, K // 16), -1, dtype=t.int32, device="cuda")
    y = lb.gemm(dev_x(inp.x), words, dev_scales(inp.scales), g, 2)
    t.cuda.synchronize()
    assert not y.float().abs().sum().item()


@pytest.mark.parametrize("bits,g", [(2, 64), (1, 128), (1, 64), (2, 32), (1, 32)])
def test_linearity_bit_exact(bits, g):
    M, N, K = 16, 512, 2048
    inp = _inputs(M, N, K, g, bits, seed=6)
    y, _ = run_gemm(inp, g, bits)
    y4, _ = run_gemm(W.Inputs(inp.x, inp.codes, (inp.scales.astype(np.float32) * 4).astype(np.float16)), g, bits)
    assert np.array_equal(oracle.bf16_bits_to_f64(y4), 4 * oracle.bf16_bits_to_f64(y))
    yn, _ = run_gemm(W.Inputs(inp.x ^ np.uint16(0x8000), inp.codes, inp.scales), g, bits)
    assert np.array_equal(oracle.bf16_bits_to_f64(yn), -oracle.bf16_bits_to_f64(y))


def test_deterministic_and_stripe_independent(monkeypatch):
    """Bitwise equal across runs; the reduction order does not depend on the stripe width."""
    inp = _inputs(16, 3072, 3072, 64, 2, seed=7)
    outs = []
    for ncb in (1, 2, 4, 4):
        monkeypatch.setenv("LOWBIT_SKINNY_NCB", str(ncb))
        y, _ = run_gemm(inp, 64, 2)
        outs.append(y)
    for y in outs[1:]:
        assert np.array_equal(y, outs[0])


def test_matches_tile_kernel_within_tolerance(monkeypatch):
    inp = _inputs(16, 3072, 3072, 64, 2, seed=8)
    ys, _ = run_gemm(inp, 64, 2)
    monkeypatch.setenv("LOWBIT_VARIANT", "tile64")
    yt, _ = run_gemm(inp, 64, 2)
    ref = oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, 64)
    assert oracle.check_tolerance(ys, ref)["ok"] and oracle.check_tolerance(yt, ref)["ok"]
