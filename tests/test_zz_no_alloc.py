"""GPU test of lowbit_gemm_noalloc (the entry point for callers that cannot allocate): through
the C-ABI it gives bitwise lowbit_gemm_ex's result (the same kernels on the library's static
scratch instead of a caller workspace) and meets the oracle, on consecutive calls whose second
input is smaller, so the scratch still holds the first call's partial sums."""
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


def _case(M, N, K, g, cid, bits=2):
    t = torch()
    inp = W.make_inputs(W.Problem("noalloc", M, N, K, bits, g, cid, M + N + K), seed=3)
    x = dev_x(inp.x)
    w, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    s = dev_scales(inp.scales)
    y = t.full((M, N), float("nan"), dtype=t.bfloat16, device="cuda")
    return inp, x, w, s, y


@pytest.mark.parametrize("shapes", [
    [(16, 3072, 12288, 64), (8, 1024, 6144, 64)],     # both split; the second has fewer tiles
    [(16, 18432, 6144, 64), (5, 512, 6144, 128)],     # 128 tiles, then a g = 128 split
    [(16, 3072, 12288, 64), (16, 3072, 3072, 64)],    # a split, then a shape that needs no scratch
])
def test_noalloc_equals_gemm_ex_on_consecutive_calls(shapes):
    t = torch()
    for i, (M, N, K, g) in enumerate(shapes):
        print(f"noalloc case {M}x{N}x{K} g={g}", flush=True)
        inp, x, w, s, y = _case(M, N, K, g, cid=90 + i)
        need = lb.workspace_size(M, N, K, g, 2)
        ws = t.zeros(max(16, need), dtype=t.uint8, device="cuda")
        want = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
        t.cuda.synchronize()
        before = t.cuda.memory_allocated()
        lb.gemm_noalloc(x, w, s, g, 2, out=y)
        t.cuda.synchronize()
        assert t.cuda.memory_allocated() == before
        got = host_bits(y)
        assert np.array_equal(got, want), f"noalloc differs from lowbit_gemm_ex at {M}x{N}x{K} g={g}"
        r = oracle.check_tolerance(got, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g))
        assert r["ok"], r
        # a repeated call on the same scratch gives the same bits
        y.fill_(float("nan"))
        lb.gemm_noalloc(x, w, s, g, 2, out=y)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(y), want)


def test_noalloc_rejects_a_plan_larger_than_its_scratch(monkeypatch):
    # a forced split plan whose workspace exceeds the scratch: refused, nothing launched
    inp, x, w, s, y = _case(16, 8704, 4096, 64, cid=95)
    monkeypatch.setenv("LOWBIT_RESIDENT_PLAN", "1,16")
    assert lb.workspace_size(16, 8704, 4096, 64, 2) > lb.NOALLOC_SCRATCH_BYTES
    with pytest.raises(lb.LowbitError) as e:
        lb.gemm_noalloc(x, w, s, 64, 2, out=y)
    assert e.value.status == 6
    torch().cuda.synchronize()
    assert torch().isnan(y.float()).all().item(), "nothing may be written"


def test_noalloc_under_graph_capture():
    """The caller this entry point is for: a captured call replayed several times, with eager work
    and an eager call of another shape on the same scratch between replays, gives the eager result
    every time (the counter clear is a fill kernel, not a memset, and every partial sum is written
    before it is read)."""
    t = torch()
    inp, x, w, s, y = _case(16, 3072, 12288, 64, cid=96)
    o_inp, ox, ow, os_, oy = _case(8, 1024, 6144, 64, cid=97)
    print("noalloc graph 16x3072x12288 g=64", flush=True)
    lb.gemm_noalloc(x, w, s, 64, 2, out=y)
    t.cuda.synchronize()
    eager = host_bits(y)
    r = oracle.check_tolerance(eager, oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, 64))
    assert r["ok"], r
    st = t.cuda.Stream()  # default priority
    st.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(st):
        lb.gemm_noalloc(x, w, s, 64, 2, out=y)  # warm up on the capture stream
    t.cuda.current_stream().wait_stream(st)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        lb.gemm_noalloc(x, w, s, 64, 2, out=y)
    other = None
    for rep in range(4):
        y.fill_(float("nan"))
        lb.gemm_noalloc(ox, ow, os_, 64, 2, out=oy)  # another split on the same scratch
        t.cuda.synchronize()
        other = host_bits(oy) if other is None else other
        assert np.array_equal(host_bits(oy), other)
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(host_bits(y), eager), f"replay {rep}"
