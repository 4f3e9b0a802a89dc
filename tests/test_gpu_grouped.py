"""GPU tests of the grouped launch (lowbit_gemm_batched): one launch per kernel family over
a table of problems.  Every output must be bitwise the single-call result and within the
oracle tolerance; chunks of more problems than one launch takes, zero-size problems, mixed
kernel families and graph capture with repeated replays are covered."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _make(shapes, cid, seed0=0):
    t = torch()
    out = []
    for i, (M, N, K, g, bits) in enumerate(shapes):
        p = W.Problem("grp", M, N, K, bits, g, cid, i)
        inp = W.make_inputs(p, seed0 + i)
        x = dev_x(inp.x)
        w, _ = lb.pack(dev_codes(inp.codes), bits)
        s = dev_scales(inp.scales)
        y = t.full((M, N), float("nan"), dtype=t.bfloat16, device="cuda")
        out.append(((x, w, s, y, g, bits), inp))
    return out


def _singles(items):
    t = torch()
    res = [host_bits(lb.gemm(x, w, s, g, bits)) for (x, w, s, y, g, bits), _ in items]
    t.cuda.synchronize()
    return res


def test_mixed_families_bitwise_equal_single_calls():
    # tile problems of different M, skinny problems of different N (so the shared stripe
    # width differs from the single-call one) and another (g, bits) class in one call
    shapes = [(512, 1152, 384, 64, 2), (64, 1152, 384, 64, 2), (16, 3072, 768, 64, 2), (7, 1024, 512, 64, 2),
              (16, 2048, 1024, 128, 2), (300, 272, 384, 128, 2), (16, 1024, 1024, 128, 1), (40, 96, 256, 32, 1)]
    items = _make(shapes, cid=50)
    singles = _singles(items)
    lb.gemm_batched([a for a, _ in items])
    torch().cuda.synchronize()
    for ((x, w, s, y, g, bits), inp), single in zip(items, singles):
        yb = host_bits(y)
        assert np.array_equal(yb, single), (tuple(x.shape), w.shape[0], g, bits)
        r = oracle.check_tolerance(yb, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
        assert r["ok"], r


def test_more_problems_than_one_launch():
    # 21 problems of one class: two launches of the skinny kernel and two of the tile kernel
    shapes = [(16 if i % 2 else 96, 256 + 64 * (i % 3), 512, 64, 2) for i in range(21)]
    items = _make(shapes, cid=51)
    singles = _singles(items)
    lb.gemm_batched([a for a, _ in items])
    torch().cuda.synchronize()
    for ((x, w, s, y, g, bits), inp), single in zip(items, singles):
        assert np.array_equal(host_bits(y), single)


def test_zero_sized_problems_in_a_batch():
    t = torch()
    items = _make([(16, 512, 512, 64, 2), (64, 256, 256, 64, 2)], cid=52)
    x0 = t.zeros((0, 256), dtype=t.bfloat16, device="cuda")
    w0 = t.zeros((32, 16), dtype=t.int32, device="cuda")
    s0 = t.ones((32, 4), dtype=t.float16, device="cuda")
    y0 = t.zeros((0, 32), dtype=t.bfloat16, device="cuda")
    xk = t.zeros((5, 0), dtype=t.bfloat16, device="cuda")
    wk = t.zeros((48, 0), dtype=t.int32, device="cuda")
    sk = t.zeros((48, 0), dtype=t.float16, device="cuda")
    yk = t.full((5, 48), 3.0, dtype=t.bfloat16, device="cuda")
    singles = _singles(items)
    lb.gemm_batched([items[0][0], (x0, w0, s0, y0, 64, 2), (xk, wk, sk, yk, 64, 2), items[1][0]])
    t.cuda.synchronize()
    assert not yk.float().abs().sum().item()
    for ((x, w, s, y, g, bits), _), single in zip(items, singles):
        assert np.array_equal(host_bits(y), single)


def test_denoise_step_pairs_as_one_launch_each():
    """The double-stream blocks' image and text linears of one kind run as one grouped call
    (scaled down: M 4096 -> 512 and 512 -> 64, every dimension of the weights / 8)."""
    for (N, K) in [(9216, 3072), (3072, 3072), (18432, 3072), (3072, 9216)]:
        items = _make([(512, N // 8, K // 8, 64, 2), (64, N // 8, K // 8, 64, 2)], cid=53)
        lb.gemm_batched([a for a, _ in items])
        torch().cuda.synchronize()
        for (x, w, s, y, g, bits), inp in items:
            r = oracle.check_tolerance(host_bits(y), oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
            assert r["ok"], (N, K, r)


def test_graph_capture_replays_match_eager():
    """A captured grouped call replayed several times, with eager work and synchronisations
    in between, gives the eager result every time (the launches record no memset)."""
    t = torch()
    items = _make([(16, 3072, 1024, 64, 2), (256, 768, 512, 64, 2), (16, 1024, 2048, 128, 2)], cid=54)
    probs = [a for a, _ in items]
    lb.gemm_batched(probs)
    t.cuda.synchronize()
    eager = [host_bits(y) for (_, _, _, y, _, _) in probs]
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        lb.gemm_batched(probs)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        lb.gemm_batched(probs)
    scratch = t.randn(1 << 20, device="cuda")
    for rep in range(4):
        for (_, _, _, y, _, _) in probs:
            y.fill_(float("nan"))
        scratch.mul_(1.0001)                      # unrelated eager work between replays
        g.replay()
        t.cuda.synchronize()
        for e, (_, _, _, y, _, _) in zip(eager, probs):
            assert np.array_equal(host_bits(y), e), f"replay {rep}"
