"""GPU parity at the size limits.

Packed weights at the header's limit (N * K * bits / 8 <= 2^32 - 1 bytes): K = 2^16 with
N = 2^18 - 16 ternary rows (4 GiB - 256 KiB of packed words) or 2^19 - 16 binary rows, on the skinny
kernel and the three tile kernels.  Every weight and scale read goes through a buffer resource whose
32-bit range covers the whole matrix, and each row's offset is a 32-bit product; the rows checked
against the oracle include both sides of the 2 GiB offset and the last.  The packed words and
scales are drawn on the device (random words whose ternary fields are made valid: 11 becomes 01);
the oracle gets the checked rows of those inputs, unpacked by its own unpack.

Activations past 4 GiB (2^20 + 40 rows of 4096): row offsets pass 2^31 and 2^32 bytes."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3
K = 1 << 16


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


@pytest.mark.parametrize("M,bits,g,variant,kernel", [
    (20, 2, 64, None, "skinny"),
    (300, 2, 64, None, "tile128x256"),
    (300, 2, 64, "tile288", "tile288x192"),
    (300, 2, 64, "tile256w", "tile256x256"),
    (300, 1, 128, None, "tile128x256"),
])
def test_weights_at_the_4gib_limit(M, bits, g, variant, kernel, monkeypatch):
    t = torch()
    N = (1 << 35) // (K * bits) - 16
    row_bytes = K * bits // 8
    assert 2 ** 32 - (1 << 18) <= N * row_bytes <= 2 ** 32 - 1
    if variant is not None:
        monkeypatch.setenv("LOWBIT_VARIANT", variant)
    assert lb.variant(M, N, K, g, bits) == kernel
    print(f"weight limit {M}x{N}x{K} bits={bits} g={g} {kernel}", flush=True)
    gen = t.Generator(device="cuda")
    gen.manual_seed(1000 + M + bits)
    w = t.randint(-2 ** 31, 2 ** 31, (N, K * bits // 32), dtype=t.int32, device="cuda", generator=gen)
    if bits == 2:
        both = w & (w >> 1) & 0x55555555  # fields 11: both bits set
        w &= ~(both << 1)
        del both
    s = (t.rand((N, K // g), device="cuda", generator=gen) * 0.045 + 0.005).to(t.float16)
    x_bits = W.gen_x(W.rng_for(7, 190, M + bits), M, K)
    y = host_bits(lb.gemm(dev_x(x_bits), w, s, g, bits))
    # rows of W on both sides of the 2 GiB byte offset, tile edges, the last rows
    mid = (1 << 31) // row_bytes
    cols = np.array(sorted({0, 1, 255, 256, mid - 1, mid, mid + 1, N // 2, N - 257, N - 256, N - 2, N - 1}))
    idx = t.as_tensor(cols, device="cuda")
    words = w.index_select(0, idx).cpu().numpy().view(np.uint32)
    scales = s.index_select(0, idx).cpu().numpy()  # float16
    codes = oracle.unpack(words, K, bits)
    ref = oracle.gemm_ref_f64(x_bits, codes, scales, g)
    r = oracle.check_tolerance(y[:, cols], ref)
    assert r["ok"], r
    assert r["rel_frob"] <= REL_ALARM, r
    del w, s
    t.cuda.empty_cache()


@pytest.mark.parametrize("variant,kernel", [("tile288", "tile288x192"), ("tile256w", "tile256x256"),
                                            ("tile64", "tile64x256")])
def test_activations_past_4gib(variant, kernel, monkeypatch):
    # X of 2^20 + 40 rows of K = 4096 (8.6 GB): row offsets pass 2^31 and 2^32 bytes; each tile's
    # rows are addressed from a 64-bit base.  Ragged in M and N.
    t = torch()
    M, N, Kx, g = (1 << 20) + 40, 272, 4096, 64
    monkeypatch.setenv("LOWBIT_VARIANT", variant)
    assert lb.variant(M, N, Kx, g, 2) == kernel
    print(f"activations past 4 GiB {M}x{N}x{Kx} {kernel}", flush=True)
    inp = W.make_inputs(W.Problem("x_limit", 1, N, Kx, 2, g, 191, 0), seed=8)   # codes and scales only
    w, bad = lb.pack(dev_codes(inp.codes), 2)
    assert bad == 0
    s = dev_scales(inp.scales)
    gen = t.Generator(device="cuda")
    gen.manual_seed(8)
    x = t.randn((M, Kx), device="cuda", generator=gen).to(t.bfloat16)
    y = lb.gemm(x, w, s, g, 2)
    row_bytes = Kx * 2
    rows = sorted({0, 1, 255, 256, (1 << 31) // row_bytes - 1, (1 << 31) // row_bytes,
                   (1 << 32) // row_bytes - 1, (1 << 32) // row_bytes, M - 41, M - 40, M - 1})
    idx = t.as_tensor(rows, device="cuda")
    x_rows = x.index_select(0, idx).cpu().view(t.int16).numpy().view(np.uint16)
    y_rows = host_bits(y.index_select(0, idx))
    del x, y
    t.cuda.empty_cache()
    ref = oracle.gemm_ref_f64(x_rows, inp.codes, inp.scales, g)
    r = oracle.check_tolerance(y_rows, ref)
    assert r["ok"], r
    assert r["rel_frob"] <= REL_ALARM, r
