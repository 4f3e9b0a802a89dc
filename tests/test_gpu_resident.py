"""GPU parity of the resident kernel (skinny ternary, activations resident in LDS, every
weight load of a wave issued at once), forced with LOWBIT_VARIANT=resident, against the
oracle, through the C-ABI."""
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


@pytest.fixture(autouse=True)
def _resident(monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", "resident")


def _inputs(M, N, K, g, seed=0, cid=70):
    p = W.Problem("resident", M, N, K, 2, g, cid, (M * 7 + N * 3 + K + g) % 100000)
    return W.make_inputs(p, seed)


def _check(y_bits, inp, g, what, cols=None):
    if cols is None:
        ref = oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g)
        got = y_bits
    else:  # output column n depends on weight row n only
        ref = oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], g)
        got = y_bits[:, cols]
    r = oracle.check_tolerance(got, ref)
    assert r["ok"], f"{what}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']}"


def _sample_cols(N, rng):
    """Columns spread over every workgroup position, plus the first and last blocks."""
    c = np.unique(np.concatenate([np.arange(32), np.arange(N - 48, N), rng.choice(N, 192, replace=False)]))
    return c[(c >= 0) & (c < N)]


# (N, K): plans (column blocks per workgroup cb, K slices ks, steps per wave len) from one
# column block (ks up to 16, one step each) to nine blocks per workgroup (ks = 1, every
# step count 1..12 of a wave)
SMALL = [(16, 256), (16, 1280), (48, 3072), (64, 4096), (256, 512), (1040, 2048)]


@pytest.mark.parametrize("N,K", SMALL)
@pytest.mark.parametrize("g", [64, 128])
def test_small_shapes(N, K, g):
    assert lb.variant(16, N, K, g, 2) == "resident"
    inp = _inputs(16, N, K, g, seed=1)
    y, _ = run_gemm(inp, g, 2)
    _check(y, inp, g, f"N={N} K={K} g={g}")


@pytest.mark.parametrize("T", list(range(1, 13)))
def test_every_wave_length(T):
    # 2304 column blocks: nine per workgroup, one K slice, so a wave walks all T steps
    N, K, g = 36864, 256 * T, 64 if T % 2 else 128
    inp = _inputs(16, N, K, g, seed=2)
    y, _ = run_gemm(inp, g, 2)
    _check(y, inp, g, f"T={T}", cols=_sample_cols(N, np.random.default_rng(T)))


@pytest.mark.parametrize("N,K", [(4112, 3072), (12304, 3072), (28672, 3072), (27648, 3072), (18432, 3072),
                                 (9216, 3072), (3072, 3072), (16384, 4096)])
def test_plans_with_k_slices(N, K):
    # several column blocks per workgroup with 2..8 K slices (uneven slices included), and
    # workgroups whose last column blocks are past N
    inp = _inputs(16, N, K, 64, seed=3)
    y, _ = run_gemm(inp, 64, 2)
    _check(y, inp, 64, f"N={N} K={K}", cols=_sample_cols(N, np.random.default_rng(N)))


@pytest.mark.parametrize("M", [1, 3, 8, 15, 16])
def test_rows(M):
    inp = _inputs(M, 1040, 3072, 64, seed=4)
    y, _ = run_gemm(inp, 64, 2)
    _check(y, inp, 64, f"M={M}")


def test_one_hot_bit_exact():
    # a single nonzero code per weight row: Y[m, n] = RNE_bf16(c * s * x[m, k]) exactly
    M, N, K, g = 16, 4112, 3072, 64
    inp = _inputs(M, N, K, g, seed=5)
    rng = np.random.default_rng(5)
    codes = np.zeros((N, K), np.int8)
    ks = rng.integers(0, K, N)
    vals = rng.choice(np.array([-1, 1], np.int8), N)
    codes[np.arange(N), ks] = vals
    t = torch()
    x = dev_x(inp.x)
    w, _ = lb.pack(dev_codes(codes), 2)
    y = lb.gemm(x, w, dev_scales(inp.scales), g, 2)
    t.cuda.synchronize()
    got = host_bits(y)
    xf = inp.x.astype(np.uint32) << 16
    xf = xf.view(np.float32).astype(np.float64)
    s = inp.scales.astype(np.float64)[np.arange(N), ks // g]
    want = (vals.astype(np.float64)[None, :] * s[None, :] * xf[:, ks]).astype(np.float32)
    want_bits = (t.from_numpy(want).to(t.bfloat16).view(t.int16).numpy().view(np.uint16))
    assert np.array_equal(got, want_bits)


def test_zero_codes_and_unused_field():
    M, N, K, g = 16, 1040, 2048, 64
    inp = _inputs(M, N, K, g, seed=6)
    t = torch()
    x = dev_x(inp.x)
    s = dev_scales(inp.scales)
    for word in (0x00000000, 0xFFFFFFFF):  # all 0 codes; all fields 11 (decode as 0)
        w = t.full((N, K // 16), np.int32(np.uint32(word).view(np.int32)), dtype=t.int32, device="cuda")
        y = lb.gemm(x, w, s, g, 2)
        t.cuda.synchronize()
        assert not np.any(host_bits(y) & 0x7FFF), hex(word)


def test_deterministic_and_batched_pairs():
    # the denoise-step pairs (image and text stream, same shape) as one batched launch:
    # deterministic, within tolerance, and each problem's result equal to the oracle
    t = torch()
    K, g = 3072, 64
    for N in (9216, 18432, 3072):
        inps = [_inputs(16, N, K, g, seed=7 + i, cid=71) for i in range(2)]
        dev = []
        for inp in inps:
            w, _ = lb.pack(dev_codes(inp.codes), 2)
            dev.append((dev_x(inp.x), w, dev_scales(inp.scales), t.empty((16, N), dtype=t.bfloat16, device="cuda"),
                        g, 2))
        lb.gemm_batched(dev)
        t.cuda.synchronize()
        first = [host_bits(d[3]).copy() for d in dev]
        lb.gemm_batched(dev)
        t.cuda.synchronize()
        for i, (inp, d) in enumerate(zip(inps, dev)):
            assert np.array_equal(first[i], host_bits(d[3])), f"N={N} problem {i} not deterministic"
            _check(first[i], inp, g, f"batched N={N} problem {i}", cols=_sample_cols(N, np.random.default_rng(i)))
        y0, _ = run_gemm(inps[0], g, 2)
        y1, _ = run_gemm(inps[0], g, 2)
        assert np.array_equal(y0, y1), f"N={N} single call not deterministic"


def test_falls_back_where_not_covered():
    # K past the LDS budget (without a workspace), M past 16, binary codes, groups of 32:
    # the forced variant is not taken
    assert lb.variant(16, 3072, 12288, 64, 2) != "resident"
    assert lb.variant(17, 3072, 3072, 64, 2) != "resident"
    assert lb.variant(16, 3072, 3072, 128, 1) != "resident"
    assert lb.variant(16, 3072, 3072, 32, 2) != "resident"
    inp = _inputs(16, 3072, 12288, 64, seed=8)
    y, _ = run_gemm(inp, 64, 2)
    _check(y, inp, 64, "K=12288 fallback")


def test_long_k_that_still_fits():
    # K = 4352: 17 steps of activations (139 KB) still fit the LDS, two steps per wave
    assert lb.variant(16, 3072, 4352, 64, 2) == "resident"
    inp = _inputs(16, 3072, 4352, 64, seed=9)
    y, _ = run_gemm(inp, 64, 2)
    _check(y, inp, 64, "K=4352")
