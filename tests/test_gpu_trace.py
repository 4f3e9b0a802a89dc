"""GPU test of the LOWBIT_TRACE launch log: with LOWBIT_TRACE=1 every GEMM kernel launch writes
one line on stderr naming the kernel family, its tile or plan, g, bits, the grid and the launch's
problems, and that kernel is the one lowbit_gemm_variant names for the shape; without it the
library writes nothing."""
from __future__ import annotations

import re

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu

LINE = re.compile(r"^lowbit: (\w+) (.*) g=(\d+) bits=(\d+) grid=(\d+) block=(\d+) lds=(\d+) problems=(\S+)$")


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _family(variant: str) -> tuple[str, str]:
    """(trace family, leading tile text) of a lowbit_gemm_variant name"""
    if variant in ("resident", "skinny"):
        return variant, ""
    m = re.match(r"tile(\d+)x(\d+)(k2)?$", variant)
    assert m, variant
    tile = f"{m.group(1)}x{m.group(2)}"
    if variant in ("tile288x192", "tile256x192", "tile96x192", "tile96x192k2", "tile64x128k2"):
        return "tile16", tile
    return "tiled32", tile


def _run(M, N, K, g, bits, cid):
    inp = W.make_inputs(W.Problem("trace", M, N, K, bits, g, cid, M + N + K), seed=4)
    y = lb.gemm(dev_x(inp.x), lb.pack(dev_codes(inp.codes), bits)[0], dev_scales(inp.scales), g, bits)
    torch().cuda.synchronize()
    return inp, host_bits(y)


@pytest.mark.parametrize("M,N,K,g,bits", [(16, 3072, 3072, 64, 2), (24, 1024, 2048, 64, 2), (700, 3072, 3072, 64, 2),
                                          (1536, 3072, 3072, 64, 2), (4608, 3072, 1024, 128, 1),
                                          (300, 512, 1024, 32, 2)])
def test_trace_names_the_launched_kernel(M, N, K, g, bits, capfd, monkeypatch):
    monkeypatch.setenv("LOWBIT_TRACE", "1")
    variant = lb.variant(M, N, K, g, bits)
    capfd.readouterr()
    inp, y = _run(M, N, K, g, bits, cid=130)
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("lowbit: ")]
    assert len(lines) == 1, err
    m = LINE.match(lines[0])
    assert m, lines[0]
    family, tile = _family(variant)
    assert m.group(1) == family, (variant, lines[0])
    assert m.group(2).startswith(tile), (variant, lines[0])
    assert (int(m.group(3)), int(m.group(4))) == (g, bits)
    assert int(m.group(5)) > 0 and int(m.group(6)) % 64 == 0
    assert m.group(8) == f"{M}x{N}x{K}"
    # the traced call still computes the product
    rows = np.r_[0:min(M, 8), max(0, M - 8):M]
    r = oracle.check_tolerance(y[rows], oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, g))
    assert r["ok"], r


def test_trace_lists_every_problem_of_a_grouped_launch(capfd, monkeypatch):
    monkeypatch.setenv("LOWBIT_TRACE", "1")
    t = torch()
    probs = []
    for i, (M, N, K) in enumerate(((512, 3072, 3072), (640, 3072, 3072))):
        inp = W.make_inputs(W.Problem("trace_b", M, N, K, 2, 64, 131 + i, 0), seed=5)
        y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        probs.append((dev_x(inp.x), lb.pack(dev_codes(inp.codes), 2)[0], dev_scales(inp.scales), y, 64, 2))
    capfd.readouterr()
    lb.gemm_batched(probs)
    t.cuda.synchronize()
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("lowbit: ")]
    assert len(lines) == 1, lines
    assert LINE.match(lines[0]).group(8) == "512x3072x3072,640x3072x3072"


def test_no_trace_without_the_variable(capfd, monkeypatch):
    monkeypatch.delenv("LOWBIT_TRACE", raising=False)
    capfd.readouterr()
    _run(16, 3072, 3072, 64, 2, cid=132)
    _run(700, 3072, 3072, 64, 2, cid=133)
    assert "lowbit: " not in capfd.readouterr().err
