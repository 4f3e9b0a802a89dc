"""GPU parity of the persistent 288 x 192 tile launch: with more tiles than compute units each
workgroup loops over several tiles (virtual ids b, b + 256, ...), issuing the next tile's first
copies before the current tile's epilogue.  Ragged multi-round shapes, a grouped launch whose
tiles span problems with different K, and the fused epilogues, against the oracle; the grouped
bits equal the single calls' (which run one tile per workgroup), and repeated launches are
bitwise equal."""
from __future__ import annotations

import math

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


def _tiles(M, N, bm=288):
    return math.ceil(M / bm) * math.ceil(N / 192)


def _inputs(M, N, K, g, bits, cid):
    inp = W.make_inputs(W.Problem("persistent", M, N, K, bits, g, cid, M + N + K + g), seed=6)
    return inp, dev_x(inp.x), lb.pack(dev_codes(inp.codes), bits)[0], dev_scales(inp.scales)


def _rows(M):
    """first and last tile rows, a tile boundary, and the ragged end"""
    return np.array(sorted({0, 1, 287, 288, 289, M // 2, M - 289, M - 288, M - 2, M - 1} & set(range(M))))


@pytest.mark.parametrize("M,N,K,g,bits", [(2900, 5008, 640, 64, 2), (2900, 5008, 640, 128, 1),
                                          (1500, 9216, 256, 64, 2), (577, 27648, 128, 128, 2)])
def test_multi_round_ragged(M, N, K, g, bits, monkeypatch):
    assert _tiles(M, N) > 256
    monkeypatch.setenv("LOWBIT_VARIANT", "tile288")
    print(f"persistent {M}x{N}x{K} g={g} bits={bits}", flush=True)
    inp, x, w, s = _inputs(M, N, K, g, bits, cid=140)
    y = host_bits(lb.gemm(x, w, s, g, bits))
    rows = _rows(M)
    r = oracle.check_tolerance(y[rows], oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, g))
    assert r["ok"], r
    assert r["rel_frob"] <= 2.5e-3, r
    # every row against the oracle on a column band that crosses a tile boundary
    cols = slice(176, 208)
    ref = oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], g)
    assert oracle.check_tolerance(y[:, cols], ref)["ok"]
    assert np.array_equal(host_bits(lb.gemm(x, w, s, g, bits)), y), "not deterministic"


@pytest.mark.parametrize("variant,bm", [("tile288", 288), ("tile256n", 256)])
def test_grouped_tiles_span_problems(variant, bm, monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", variant)
    t = torch()
    shapes = [(1200, 4096, 512), (700, 6144, 1024), (2000, 2048, 256)]
    assert sum(_tiles(M, N, bm) for M, N, _ in shapes) > 256
    items = []
    for i, (M, N, K) in enumerate(shapes):
        inp, x, w, s = _inputs(M, N, K, 64, 2, cid=141 + i)
        items.append((inp, (x, w, s, t.empty((M, N), dtype=t.bfloat16, device="cuda"), 64, 2)))
    singles = [host_bits(lb.gemm(a[0], a[1], a[2], 64, 2)) for _, a in items]
    lb.gemm_batched([a for _, a in items])
    t.cuda.synchronize()
    for (inp, a), single, (M, N, K) in zip(items, singles, shapes):
        got = host_bits(a[3])
        assert np.array_equal(got, single), f"grouped {M}x{N}x{K} differs from its single call"
        rows = _rows(M)
        r = oracle.check_tolerance(got[rows], oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, 64))
        assert r["ok"], (M, N, K, r)


def test_fused_epilogues_multi_round():
    t = torch()
    # SwiGLU: 2N weight rows (gate then up), N output columns; 288 x 192 weight tiles of 96 outputs
    M, N, K, g = 1200, 6144, 384, 64
    assert math.ceil(M / 288) * (2 * N // 192) > 256
    inp = W.make_inputs(W.Problem("persistent_swiglu", M, 2 * N, K, 2, g, 144, 1), seed=7)
    x, w, s = dev_x(inp.x), lb.pack(dev_codes(inp.codes), 2)[0], dev_scales(inp.scales)
    y = host_bits(lb.gemm_swiglu(x, w, s, g, 2))
    rows = _rows(M)
    r = oracle.check_tolerance(y[rows], oracle.swiglu_ref_f64(inp.x[rows], inp.codes, inp.scales, g))
    assert r["ok"], r
    # gated residual in place: Y = R + gate * (X . W^T)
    M, N, K = 1500, 9216, 256
    rows = _rows(M)
    inp, x, w, s = _inputs(M, N, K, 64, 2, cid=145)
    rng = np.random.default_rng(3)
    R = oracle.f64_to_bf16_bits_rne(rng.standard_normal((M, N)))
    gate = oracle.f64_to_bf16_bits_rne(rng.standard_normal(N) * 0.5)
    Rd = t.from_numpy(R.view(np.int16)).cuda().view(t.bfloat16)
    gd = t.from_numpy(gate.view(np.int16)).cuda().view(t.bfloat16)
    lb.gemm_residual(x, w, s, 64, 2, Rd, gd, out=Rd)
    t.cuda.synchronize()
    got = host_bits(Rd)
    r = oracle.check_tolerance(got[rows], oracle.residual_ref_f64(inp.x[rows], inp.codes, inp.scales, 64, R[rows], gate))
    assert r["ok"], r


@pytest.mark.parametrize("M,N,K,g", [(288, 192 * 257, 128, 64),          # 257 tiles: one workgroup runs two
                                     (7 * 288, 73 * 192, 128, 64),       # 511 tiles: one workgroup runs one
                                     (16 * 288, 32 * 192, 64, 64),       # 512 tiles, a single K step each
                                     (27 * 288 - 5, 19 * 192 - 16, 128, 128)])  # 513 tiles, ragged edges
def test_tile_counts_around_whole_rounds(M, N, K, g, monkeypatch):
    """Tile counts one below, at and one above a multiple of the 256 workgroups: the loop's exit
    (next virtual id past the tile count) on every workgroup, and the last round's odd tile."""
    monkeypatch.setenv("LOWBIT_VARIANT", "tile288")
    print(f"persistent edges {M}x{N}x{K} g={g} tiles={_tiles(M, N)}", flush=True)
    inp, x, w, s = _inputs(M, N, K, g, 2, cid=146)
    y = host_bits(lb.gemm(x, w, s, g, 2))
    rows = _rows(M)
    r = oracle.check_tolerance(y[rows], oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, g))
    assert r["ok"], r
    # the last tile (highest virtual id) in full
    r0, c0 = ((M - 1) // 288) * 288, ((N - 1) // 192) * 192
    ref = oracle.gemm_ref_f64(inp.x[r0:], inp.codes[c0:], inp.scales[c0:], g)
    assert oracle.check_tolerance(y[r0:, c0:], ref)["ok"]


@pytest.mark.parametrize("g,bits", [(64, 2), (128, 1)])
def test_256x192_multi_round_ragged(g, bits, monkeypatch):
    """The 256 x 192 tile (12 waves of 128 x 32) persistent over three rounds, with a ragged last
    row and column of tiles."""
    M, N, K = 4096 - 7, 9216 - 16, 384
    assert math.ceil(M / 256) * math.ceil(N / 192) == 768
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256n")
    assert lb.variant(M, N, K, g, bits) == "tile256x192"
    print(f"persistent 256x192 {M}x{N}x{K} g={g} bits={bits}", flush=True)
    inp, x, w, s = _inputs(M, N, K, g, bits, cid=147)
    y = host_bits(lb.gemm(x, w, s, g, bits))
    rows = np.array(sorted({0, 1, 255, 256, 257, 2047, 2048, M - 250, M - 1}))
    r = oracle.check_tolerance(y[rows], oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, g))
    assert r["ok"], r
    cols = slice(N - 200, N)  # the ragged last column of tiles and its neighbour
    assert oracle.check_tolerance(y[:, cols], oracle.gemm_ref_f64(inp.x, inp.codes[cols], inp.scales[cols], g))["ok"]
