"""GPU parity of the ring kernel (skinny ternary, deep LDS load ring) and of its split-K
through a caller workspace (lowbit_gemm_ex), against the oracle, through the C-ABI."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, run_gemm, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _inputs(M, N, K, g, seed=0, cid=60):
    p = W.Problem("ring", M, N, K, 2, g, cid, (M * 7 + N * 3 + K + g) % 100000)
    return W.make_inputs(p, seed)


def _dev(inp):
    x = dev_x(inp.x)
    w, bad = lb.pack(dev_codes(inp.codes), 2)
    assert bad == 0
    return x, w, dev_scales(inp.scales)


def _check(y_bits, inp, g, what):
    r = oracle.check_tolerance(y_bits, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
    assert r["ok"], f"{what}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']}"


def _workspace(M, N, K, g):
    t = torch()
    n = lb.workspace_size(M, N, K, g, 2)
    return t.zeros(max(n, 16), dtype=t.uint8, device="cuda"), n


@pytest.mark.parametrize("K", [256, 512, 768, 1024, 1280, 2048, 3072])
@pytest.mark.parametrize("g", [64, 128])
def test_ring_without_split_every_step_count(K, g, monkeypatch):
    # one workgroup walks all K steps: the main loop of 4 steps and every remainder 0..3
    monkeypatch.setenv("LOWBIT_VARIANT", "ring")
    for N in (128, 192):  # two-block and one-block column tiles
        inp = _inputs(16, N, K, g, seed=1)
        y, _ = run_gemm(inp, g, 2)
        _check(y, inp, g, f"ring N={N} K={K} g={g}")


@pytest.mark.parametrize("M", [1, 3, 8, 15, 16])
def test_ring_rows(M, monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", "ring")
    inp = _inputs(M, 640, 1536, 64, seed=2)
    y, _ = run_gemm(inp, 64, 2)
    _check(y, inp, 64, f"ring M={M}")


@pytest.mark.parametrize("max_splits", [2, 3, 4, 16])
@pytest.mark.parametrize("g", [64, 128])
def test_split_k_through_workspace(max_splits, g, monkeypatch):
    monkeypatch.setenv("LOWBIT_RING_MAX_SPLITS", str(max_splits))
    M, N, K = 16, 512, 3072          # few column tiles: the plan splits K as far as allowed
    inp = _inputs(M, N, K, g, seed=3)
    x, w, s = _dev(inp)
    ws, n = _workspace(M, N, K, g)
    assert n > 0
    y1 = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
    _check(y1, inp, g, f"split<= {max_splits}")
    # the call leaves the counters at zero: the same workspace gives bitwise the same result
    y2 = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
    torch().cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert not ws[: 256].any().item(), "arrival counters not reset"


def test_split_k_shapes_of_the_denoise_step():
    for (N, K) in [(3072, 3072), (3072, 9216), (3072, 12288), (9216, 3072)]:
        inp = _inputs(16, N, K, 64, seed=4)
        x, w, s = _dev(inp)
        ws, n = _workspace(16, N, K, 64)
        y = host_bits(lb.gemm(x, w, s, 64, 2, workspace=ws))
        _check(y, inp, 64, f"ex {N}x{K} ws={n}")


def test_ex_falls_back_without_enough_workspace():
    t = torch()
    M, N, K = 16, 512, 3072
    inp = _inputs(M, N, K, 64, seed=5)
    x, w, s = _dev(inp)
    plain = host_bits(lb.gemm(x, w, s, 64, 2))
    small = t.zeros(64, dtype=t.uint8, device="cuda")
    assert np.array_equal(host_bits(lb.gemm(x, w, s, 64, 2, workspace=small)), plain)
    # shapes the ring kernel does not take need no workspace and equal lowbit_gemm
    for (MM, g, bits) in ((32, 64, 2), (16, 64, 1), (16, 32, 2)):
        assert lb.workspace_size(MM, N, K, g, bits) == 0
        p = W.Problem("fb", MM, N, K, bits, g, 61, MM + g + bits)
        inp2 = W.make_inputs(p, 6)
        x2 = dev_x(inp2.x)
        w2, _ = lb.pack(dev_codes(inp2.codes), bits)
        s2 = dev_scales(inp2.scales)
        a = host_bits(lb.gemm(x2, w2, s2, g, bits))
        b = host_bits(lb.gemm(x2, w2, s2, g, bits, workspace=small))
        assert np.array_equal(a, b)


def test_ring_one_hot_bit_exact(monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", "ring")
    M, N, K, g = 16, 256, 1024, 64
    x = W.gen_x(W.rng_for(4, 62, 0), M, K)
    s = W.gen_scales(W.rng_for(4, 62, 1), N, K, g)
    xf = oracle.bf16_bits_to_f64(x)
    for (n0, k0, c0) in ((0, 0, 1), (63, 255, -1), (64, 256, 1), (255, 1023, -1), (130, 517, 1)):
        c = np.zeros((N, K), dtype=np.int8)
        c[n0, k0] = c0
        y, _ = run_gemm(W.Inputs(x, c, s), g, 2)
        want = oracle.f64_to_bf16_bits_rne(c0 * float(s[n0, k0 // g]) * xf[:, k0])
        col = y[:, n0]
        zero = lambda b: (b & 0x7FFF) == 0
        assert ((col == want) | (zero(col) & zero(want))).all(), (n0, k0)
        assert np.all(zero(np.delete(y, n0, axis=1)))


def test_ring_deterministic_and_default_choice():
    # N = 27648 fills the machine without splitting K: lowbit_gemm picks the ring kernel
    assert lb.variant(16, 27648, 3072, 64, 2) == "ring"
    inp = _inputs(16, 27648, 3072, 64, seed=7)
    y1, _ = run_gemm(inp, 64, 2)
    y2, _ = run_gemm(inp, 64, 2)
    assert np.array_equal(y1, y2)
    rows = np.arange(16)
    cols = np.random.default_rng(0).choice(27648, 2048, replace=False)
    ref = oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], 64)
    _check(y1[:, cols], W.Inputs(inp.x, inp.codes[cols], inp.scales[cols]), 64, "N=27648 sampled columns")
