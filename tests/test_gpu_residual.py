"""GPU parity of the gated-residual entry point (lowbit_gemm_residual: Y = R + gate[n] * (X . W^T))
against the oracle, through the C-ABI, with its exact special cases."""
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


def _case(M, N, K, g, bits, seed=0):
    """Inputs, the residual R [M, N] and the gate [N] (bf16 bit patterns, N(0,1) like X)."""
    p = W.Problem("residual", M, N, K, bits, g, 91, (M * 7 + N * 5 + K + g + bits) % 100000)
    inp = W.make_inputs(p, seed)
    rng = np.random.default_rng(seed + 1000)
    r = W.gen_x(rng, M, N)
    gt = W.gen_x(rng, 1, N)[0]
    return inp, r, gt


def _dev(inp, bits):
    x = dev_x(inp.x)
    words, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    return x, words, dev_scales(inp.scales)


def _bits_to_dev(b):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(t.bfloat16).cuda()


def _check(y_bits, ref, what):
    r = oracle.check_tolerance(y_bits, ref)
    assert r["ok"], f"{what}: {r}"
    floor = oracle.check_tolerance(oracle.f64_to_bf16_bits_rne(ref), ref)["rel_frob"]
    assert r["rel_frob"] <= max(REL_ALARM, 1.5 * floor), f"{what}: rel_frob {r['rel_frob']} (floor {floor})"


# large M on the 16x16-block tile kernel (ragged M and N, one step to many, g 64 / 128, both bit
# widths); skinny ternary M on the resident kernel, or the tile kernel where K does not fit
SHAPES = [(300, 400, 1280, 64, 2), (577, 208, 3072, 128, 1), (289, 1008, 2304, 64, 2), (1, 16, 64, 64, 2),
          (16, 3072, 3072, 64, 2), (7, 400, 1280, 128, 2), (16, 3072, 12288, 64, 2), (16, 208, 512, 64, 1)]


@pytest.mark.parametrize("M,N,K,g,bits", SHAPES)
def test_residual_parity(M, N, K, g, bits):
    inp, r, gt = _case(M, N, K, g, bits)
    x, w, s = _dev(inp, bits)
    y = host_bits(lb.gemm_residual(x, w, s, g, bits, _bits_to_dev(r), _bits_to_dev(gt)))
    _check(y, oracle.residual_ref_f64(inp.x, inp.codes, inp.scales, g, r, gt), f"residual {M}x{N}x{K} g{g} b{bits}")


@pytest.mark.parametrize("M,N,K,kernel", [(300, 400, 1280, "tile288"), (16, 3072, 3072, "resident")])
def test_residual_special_gates_bit_exact(M, N, K, kernel, monkeypatch):
    """gate = 0 returns R bit for bit; R = 0 and gate = 1 return the bits of lowbit_gemm on the same
    kernel (fp32: 0 * v + r is r and 1 * v + 0 is v, exactly)."""
    monkeypatch.setenv("LOWBIT_VARIANT", kernel)  # lowbit_gemm on the kernel the epilogue runs on
    t = torch()
    g, bits = 64, 2
    inp, r, _ = _case(M, N, K, g, bits, seed=3)
    x, w, s = _dev(inp, bits)
    R = _bits_to_dev(r)
    y0 = host_bits(lb.gemm_residual(x, w, s, g, bits, R, t.zeros(N, dtype=t.bfloat16, device="cuda")))
    assert np.array_equal(y0, r)
    y1 = host_bits(lb.gemm_residual(x, w, s, g, bits, t.zeros((M, N), dtype=t.bfloat16, device="cuda"),
                                    t.ones(N, dtype=t.bfloat16, device="cuda")))
    assert np.array_equal(y1, host_bits(lb.gemm(x, w, s, g, bits)))


@pytest.mark.parametrize("M,N,K", [(300, 400, 1280), (16, 3072, 3072)])
def test_residual_in_place(M, N, K):
    """Y may be R: the in-place update gives the out-of-place bits."""
    g, bits = 64, 2
    inp, r, gt = _case(M, N, K, g, bits, seed=4)
    x, w, s = _dev(inp, bits)
    G = _bits_to_dev(gt)
    out_of_place = host_bits(lb.gemm_residual(x, w, s, g, bits, _bits_to_dev(r), G))
    R = _bits_to_dev(r)
    lb.gemm_residual(x, w, s, g, bits, R, G, out=R)
    assert np.array_equal(host_bits(R), out_of_place)


def test_residual_proj_full_size_sampled():
    """The proj linear at 1024^2 (M = 4608, 3072 x 3072, ternary g = 64) with a gated residual,
    in the launch configuration bench.py times; sampled rows against the oracle."""
    M, N, K, g, bits = 4608, 3072, 3072, 64, 2
    inp, r, gt = _case(M, N, K, g, bits, seed=5)
    x, w, s = _dev(inp, bits)
    y = host_bits(lb.gemm_residual(x, w, s, g, bits, _bits_to_dev(r), _bits_to_dev(gt)))
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                     np.random.default_rng(1).choice(M, 48, replace=False)]))
    ref = oracle.residual_ref_f64(inp.x[rows], inp.codes, inp.scales, g, r[rows], gt)
    _check(y[rows], ref, "residual 4608x3072x3072 (sampled rows)")


def test_residual_k0_and_rejects():
    t = torch()
    x0 = t.zeros((5, 0), dtype=t.bfloat16, device="cuda")
    w0 = t.zeros((32, 0), dtype=t.int32, device="cuda")
    s0 = t.zeros((32, 0), dtype=t.float16, device="cuda")
    R = t.randn((5, 32), device="cuda").to(t.bfloat16)
    G = t.randn(32, device="cuda").to(t.bfloat16)
    y = lb.gemm_residual(x0, w0, s0, 64, 2, R, G)
    assert t.equal(y, R)
    x = t.zeros((4, 64), dtype=t.bfloat16, device="cuda")
    w = t.zeros((32, 4), dtype=t.int32, device="cuda")
    s = t.ones((32, 2), dtype=t.float16, device="cuda")
    with pytest.raises(lb.LowbitError):
        lb.gemm_residual(x, w, s, 32, 2, t.zeros((4, 32), dtype=t.bfloat16, device="cuda"), G)
    with pytest.raises(ValueError):
        lb.gemm_residual(x, w, s[:, :1], 64, 2, t.zeros((4, 16), dtype=t.bfloat16, device="cuda"), G)
