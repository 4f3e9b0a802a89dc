"""GPU parity at long K, up to the header's limit K <= 2^22: the tile kernels (ternary and binary)
and the skinny-M path at K = 2^20, and K = 2^22 itself.  Over 16384 scale groups the fp32 sums
stay within the tolerance, and no byte offset (activation rows of 2 or 8 MiB, weight rows of 256 KiB
or 1 MiB) wraps."""
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


@pytest.mark.parametrize("M,N,K,g,bits,rows,variant", [
    (300, 48, 1 << 20, 64, 2, (0, 149, 288, 299), None),         # 64 x 256 tiles, five rows of them
    (300, 48, 1 << 20, 64, 2, (0, 149, 287, 288, 299), "tile288"),  # the 16x16-block kernel
    (300, 48, 1 << 20, 128, 1, (0, 150, 255, 256, 299), "tile256w"),  # 256 x 256, binary g = 128
    (16, 64, 1 << 20, 64, 2, None, None),                          # skinny M, every row
    (2, 16, 1 << 22, 64, 2, None, None),                           # the longest K the header allows
])
def test_long_k(M, N, K, g, bits, rows, variant, monkeypatch):
    if variant is not None:
        monkeypatch.setenv("LOWBIT_VARIANT", variant)
    print(f"long K {M}x{N}x{K} g={g} bits={bits} variant={lb.variant(M, N, K, g, bits)}", flush=True)
    inp = W.make_inputs(W.Problem("long_k", M, N, K, bits, g, 160, K.bit_length()), seed=5)
    w, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    y = host_bits(lb.gemm(dev_x(inp.x), w, dev_scales(inp.scales), g, bits))
    sel = np.arange(M) if rows is None else np.array(rows)
    r = oracle.check_tolerance(y[sel], oracle.gemm_ref_f64(inp.x[sel], inp.codes, inp.scales, g))
    assert r["ok"], r
    assert r["rel_frob"] <= REL_ALARM, r
