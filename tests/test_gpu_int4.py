"""GPU parity of 4-bit codes (two's complement nibbles, w = s * c with c in [-8, 7]) against the
oracle, through the C-ABI: pack / unpack bit-exact, lowbit_gemm on every 16x16-block tile
variant, the text encoder's MLP linears at full size, the fused epilogues and a batched call."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, host_words, run_gemm, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _inputs(M, N, K, g, seed=0):
    p = W.Problem("int4", M, N, K, 4, g, 93, (M * 3 + N * 7 + K + g) % 100000)
    return W.make_inputs(p, seed)


def _check(y_bits, ref, what):
    r = oracle.check_tolerance(y_bits, ref)
    assert r["ok"], f"{what}: {r}"
    floor = oracle.check_tolerance(oracle.f64_to_bf16_bits_rne(ref), ref)["rel_frob"]
    assert r["rel_frob"] <= max(REL_ALARM, 1.5 * floor), f"{what}: rel_frob {r['rel_frob']} (floor {floor})"


@pytest.mark.parametrize("N,K", [(16, 8), (208, 1040), (3072, 2560)])
def test_int4_pack_unpack_bit_exact(N, K):
    rng = np.random.default_rng(N + K)
    codes = W.gen_codes(rng, N, K, 4)
    codes[0, :min(K, 16)] = np.arange(-8, 8)[:min(K, 16)]
    codes.flat[rng.choice(N * K, 5, replace=False)] = np.array([8, -9, 127, -128, 20], dtype=np.int8)
    words, bad = lb.pack(dev_codes(codes), 4)
    want, want_bad = oracle.pack(codes, 4)
    assert bad == want_bad == 5 and np.array_equal(host_words(words), want)
    back = lb.unpack(words, K, 4).cpu().numpy()
    assert np.array_equal(back, oracle.unpack(want, K, 4))


# ragged M and N, one K step to many (K = 8448 is 132 steps), g = 64 / 128
SHAPES = [(300, 400, 1280, 64), (577, 208, 3072, 128), (1, 16, 64, 64), (16, 3072, 2560, 64), (289, 1008, 2304, 128),
          (96, 112, 8448, 64)]


@pytest.mark.parametrize("M,N,K,g", SHAPES)
def test_int4_gemm_parity(M, N, K, g):
    inp = _inputs(M, N, K, g)
    y, _ = run_gemm(inp, g, 4)
    _check(y, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g), f"int4 {M}x{N}x{K} g{g}")


@pytest.mark.parametrize("variant", ["tile288", "tile256n", "tile96", "tile96k2", "tile64k2"])
@pytest.mark.parametrize("g", [64, 128])
def test_int4_every_tile_variant(variant, g, monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", variant)
    M, N, K = 200, 400, 1536  # 24 steps: even, so tile96k2 splits K
    assert lb.variant(M, N, K, g, 4) == {"tile288": "tile288x192", "tile256n": "tile256x192", "tile96": "tile96x192",
                                         "tile96k2": "tile96x192k2", "tile64k2": "tile64x128k2"}[variant]
    inp = _inputs(M, N, K, g, seed=3)
    y, _ = run_gemm(inp, g, 4)
    _check(y, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g), f"int4 {variant} g{g}")


def test_int4_one_hot_bit_exact():
    """One code c at (n0, k0): Y[:, n0] is the bf16 rounding of the exact c * s * x (the kernel's
    16c * x and its product with s / 16 are exact in fp32), every other column exactly 0."""
    M, N, K, g = 40, 208, 512, 64
    rng = W.rng_for(1, 97, 0)
    x = W.gen_x(rng, M, K)
    s = W.gen_scales(rng, N, K, g)
    xd, sd = dev_x(x), dev_scales(s)
    xf = oracle.bf16_bits_to_f64(x)
    for (n0, k0, c0) in ((0, 0, -8), (207, 511, 7), (100, 200, -3), (17, 63, 5)):
        c = np.zeros((N, K), dtype=np.int8)
        c[n0, k0] = c0
        words, _ = lb.pack(dev_codes(c), 4)
        y = host_bits(lb.gemm(xd, words, sd, g, 4))
        want = oracle.f64_to_bf16_bits_rne(c0 * float(s[n0, k0 // g]) * xf[:, k0])
        assert np.array_equal(y[:, n0], want), (n0, k0, c0)
        assert not np.any(np.delete(y, n0, axis=1) & 0x7FFF)


@pytest.mark.parametrize("N,K", [(19456, 2560), (2560, 9728)])
def test_int4_text_encoder_mlp_full_size_sampled(N, K):
    """The 4-bit text encoder's MLP linears at a 512-token prompt (hidden 2560, intermediate
    9728: gate and up fused into 19456 outputs, and down), in the launch configuration bench.py
    times; sampled output columns against the oracle."""
    M, g = 512, 64
    inp = _inputs(M, N, K, g, seed=5)
    y, _ = run_gemm(inp, g, 4)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                     np.random.default_rng(2).choice(N, 64, replace=False)]))
    ref = oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], g)
    _check(y[:, cols], ref, f"int4 512x{N}x{K} (sampled)")


def test_int4_swiglu_and_residual():
    t = torch()
    M, N, K, g = 300, 208, 1280, 64
    p = W.Problem("int4_swiglu", M, 2 * N, K, 4, g, 94, 11)
    inp = W.make_inputs(p, 0)
    x = dev_x(inp.x)
    words, bad = lb.pack(dev_codes(inp.codes), 4)
    s = dev_scales(inp.scales)
    y = host_bits(lb.gemm_swiglu(x, words, s, g, 4))
    _check(y, oracle.swiglu_ref_f64(inp.x, inp.codes, inp.scales, g), "int4 swiglu")
    rng = np.random.default_rng(12)
    r, gt = W.gen_x(rng, M, 2 * N), W.gen_x(rng, 1, 2 * N)[0]
    dev = lambda b: t.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(t.bfloat16).cuda()
    y = host_bits(lb.gemm_residual(x, words, s, g, 4, dev(r), dev(gt)))
    _check(y, oracle.residual_ref_f64(inp.x, inp.codes, inp.scales, g, r, gt), "int4 residual")


def test_int4_in_a_batched_call_with_ternary():
    """A batched call holding 4-bit and ternary problems: each class gets its own launch."""
    t = torch()
    cases = [(_inputs(96, 400, 1280, 64, seed=8), 4), (W.make_inputs(W.Problem("t", 64, 208, 512, 2, 64, 95, 3), 0), 2),
             (_inputs(17, 3072, 2560, 128, seed=9), 4)]
    probs, outs = [], []
    for inp, bits in cases:
        g = inp.scales.shape[1] and inp.codes.shape[1] // inp.scales.shape[1]
        words, _ = lb.pack(dev_codes(inp.codes), bits)
        out = t.empty((inp.x.shape[0], inp.codes.shape[0]), dtype=t.bfloat16, device="cuda")
        probs.append((dev_x(inp.x), words, dev_scales(inp.scales), out, g, bits))
        outs.append((out, inp, g))
    lb.gemm_batched(probs)
    for out, inp, g in outs:
        _check(host_bits(out), oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g), "batched")


def test_int4_empty_and_k0():
    """M = 0 is a no-op, K = 0 gives Y = 0 (every output overwritten), N = 0 packs nothing."""
    t = torch()
    x0 = t.zeros((5, 0), dtype=t.bfloat16, device="cuda")
    w0 = t.zeros((32, 0), dtype=t.int32, device="cuda")
    s0 = t.zeros((32, 0), dtype=t.float16, device="cuda")
    y = t.full((5, 32), 3.0, dtype=t.bfloat16, device="cuda")
    lb.gemm(x0, w0, s0, 64, 4, out=y)
    assert not y.float().abs().sum().item()
    x = t.zeros((0, 64), dtype=t.bfloat16, device="cuda")
    w = t.zeros((32, 8), dtype=t.int32, device="cuda")
    s = t.ones((32, 1), dtype=t.float16, device="cuda")
    assert lb.gemm(x, w, s, 64, 4).shape == (0, 32)
    words, bad = lb.pack(t.zeros((0, 64), dtype=t.int8, device="cuda"), 4)
    assert words.shape == (0, 8) and bad == 0
