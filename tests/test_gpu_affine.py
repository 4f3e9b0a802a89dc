"""GPU parity of the affine 4-bit path (lowbit_pack_u4, lowbit_gemm_affine: w = s * q + b with
unsigned levels q in 0 .. 15 and an fp16 scale and bias per group) against the oracle, through the
C-ABI: bit-exact packing, every 16x16-block tile at g = 64 and 128 on ragged shapes, exact one-hot
products of the scale and of the bias path, the text encoder's MLP linears at full size, and the
edge cases."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_scales, dev_x, host_bits, host_words, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _problem(M, N, K, g, cid=120):
    return W.Problem("affine", M, N, K, W.INT4, g, cid, (M * 7 + N * 3 + K + g) % 100000, affine=True)


def _dev_levels(q):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(q, dtype=np.uint8)).cuda()


def _run(inp, g, out=None):
    words, bad = lb.pack_u4(_dev_levels(inp.codes))
    assert bad == 0
    y = lb.gemm_affine(dev_x(inp.x), words, dev_scales(inp.scales), dev_scales(inp.biases), g, out=out)
    torch().cuda.synchronize()
    return host_bits(y), words


def _check(y_bits, inp, g, what, rows=None):
    x = inp.x if rows is None else inp.x[rows]
    yref = oracle.gemm_affine_ref_f64(x, inp.codes, inp.scales, inp.biases, g)
    r = oracle.check_tolerance(y_bits if rows is None else y_bits[rows], yref)
    assert r["ok"], f"{what}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']} above alarm"


@pytest.mark.parametrize("N,K", [(16, 64), (272, 320), (1008, 4352), (2560, 512)])
def test_pack_u4_bit_exact(N, K):
    q = W.gen_levels(W.rng_for(1, 121, N + K), N, K).astype(np.uint8)
    q[0, :16] = np.arange(16)
    words, bad = lb.pack_u4(_dev_levels(q))
    want, _ = oracle.pack_u4(q)
    assert bad == 0
    assert np.array_equal(host_words(words), want)


def test_pack_u4_counts_invalid_levels():
    q = np.zeros((16, 64), dtype=np.uint8)
    q[3, 5], q[7, 63], q[15, 0], q[0, 1] = 16, 255, 200, 15
    words, bad = lb.pack_u4(_dev_levels(q))
    want, want_bad = oracle.pack_u4(q)
    assert bad == want_bad == 3
    assert np.array_equal(host_words(words), want)


# ragged M and N, one K step to many, both group sizes
@pytest.mark.parametrize("M,N,K,g", [(1, 16, 64, 64), (37, 272, 320, 64), (300, 400, 1024, 128),
                                     (577, 1040, 2560, 64), (64, 256, 8448, 128), (290, 208, 128, 64)])
def test_affine_matches_oracle(M, N, K, g):
    inp = W.make_inputs(_problem(M, N, K, g), seed=2)
    y, _ = _run(inp, g)
    _check(y, inp, g, f"affine {M}x{N}x{K} g{g}")


@pytest.mark.parametrize("variant", ["tile288", "tile256n", "tile96", "tile96k2", "tile64k2"])
@pytest.mark.parametrize("g", [64, 128])
def test_every_tile_variant(variant, g, monkeypatch):
    monkeypatch.setenv("LOWBIT_VARIANT", variant)
    M, N, K = 200, 400, 1024  # K / 64 even: the K-split tiles split
    inp = W.make_inputs(_problem(M, N, K, g, cid=122), seed=3)
    y, _ = _run(inp, g)
    _check(y, inp, g, f"{variant} g{g}")
    y2, _ = _run(inp, g)
    assert np.array_equal(y, y2), "not deterministic"


def test_one_hot_level_is_exact():
    """One nonzero level q at (n0, k0), zero biases: Y[:, n0] = RNE_bf16(q * s * x[:, k0]) exactly
    (q * s * x has at most 4 + 11 + 8 significant bits, exact in fp32), every other column 0."""
    M, N, K, g = 40, 64, 256, 64
    inp = W.make_inputs(_problem(M, N, K, g, cid=123), seed=4)
    xf = oracle.bf16_bits_to_f64(inp.x)
    b = np.zeros_like(inp.biases)
    for (n0, k0, q0) in ((0, 0, 15), (63, 255, 1), (17, 130, 9), (40, 64, 8)):
        q = np.zeros((N, K), dtype=np.uint8)
        q[n0, k0] = q0
        y, _ = _run(W.Inputs(inp.x, q, inp.scales, b), g)
        want = oracle.f64_to_bf16_bits_rne(q0 * float(inp.scales[n0, k0 // g]) * xf[:, k0])
        assert np.array_equal(y[:, n0], want), (n0, k0)
        assert not np.any(np.delete(y, n0, axis=1) & 0x7FFF)


@pytest.mark.parametrize("variant", [None, "tile288", "tile256n", "tile96", "tile96k2", "tile64k2"])
def test_one_hot_bias_is_exact(variant, monkeypatch):
    """Zero scales, one nonzero bias b at (n0, group j) and one nonzero activation per row at k0
    in group j: Y[:, n0] = RNE_bf16(b * x[:, k0]) exactly (the bias path's activation sum of a
    single element), every other column 0; on every tile (fp32 FMAs per group on the 12-wave
    tile, a bias MFMA per four groups on the others)."""
    if variant is not None:
        monkeypatch.setenv("LOWBIT_VARIANT", variant)
    M, N, K, g = 24, 48, 384, 128
    inp = W.make_inputs(_problem(M, N, K, g, cid=124), seed=5)
    s = np.zeros_like(inp.scales)
    for (n0, k0) in ((0, 0), (47, 383), (20, 200)):
        x = np.zeros_like(inp.x)
        x[:, k0] = inp.x[:, k0]
        b = np.zeros_like(inp.biases)
        b[n0, k0 // g] = inp.biases[n0, k0 // g]
        y, _ = _run(W.Inputs(x, inp.codes, s, b), g)
        want = oracle.f64_to_bf16_bits_rne(float(b[n0, k0 // g]) * oracle.bf16_bits_to_f64(x[:, k0]))
        assert np.array_equal(y[:, n0], want), (n0, k0)
        assert not np.any(np.delete(y, n0, axis=1) & 0x7FFF)


@pytest.mark.parametrize("variant", ["tile288", "tile256n", "tile96", "tile96k2", "tile64k2"])
@pytest.mark.parametrize("K,g", [(384, 64), (384, 128), (1408, 64), (1408, 128), (64, 64)])
def test_bias_sets_across_k_groups(variant, K, g, monkeypatch):
    """The bias terms of sets of four groups: K ranges that start or end inside a set (K split
    between two groups of waves at 3 or 11 steps each, g = 128 splitting a group between them),
    several full sets, a single step, ragged M and N."""
    monkeypatch.setenv("LOWBIT_VARIANT", variant)
    M, N = 100, 208
    inp = W.make_inputs(_problem(M, N, K, g, cid=128), seed=8)
    y, _ = _run(inp, g)
    _check(y, inp, g, f"bias sets {variant} K={K} g{g}")


def test_shifted_symmetric_weights_match_the_int4_path():
    """b = -8 s and q = c + 8 is the symmetric 4-bit weight s * c: both entry points meet the same
    oracle result."""
    M, N, K, g = 96, 192, 512, 64
    p = W.Problem("sym", M, N, K, W.INT4, g, 125, 1)
    inp = W.make_inputs(p, seed=6)
    b = (np.float16(-8.0) * inp.scales).astype(np.float16)
    yref = oracle.gemm_ref_f64(inp.x, inp.codes, inp.scales, g)
    y_aff, _ = _run(W.Inputs(inp.x, (inp.codes.astype(np.int16) + 8).astype(np.uint8), inp.scales, b), g)
    r = oracle.check_tolerance(y_aff, yref)
    assert r["ok"] and r["rel_frob"] <= REL_ALARM, r
    words, _ = lb.pack(torch().from_numpy(inp.codes).cuda(), 4)
    y_sym = host_bits(lb.gemm(dev_x(inp.x), words, dev_scales(inp.scales), g, 4))
    assert oracle.check_tolerance(y_sym, yref)["ok"]


@pytest.mark.parametrize("name,N,K", [("te_mlp_gate_up", 19456, 2560), ("te_mlp_down", 2560, 9728)])
def test_text_encoder_mlp_full_size(name, N, K):
    """The text encoder's MLP linears (hidden 2560, intermediate 9728) at a 512-token prompt, all
    columns of sampled rows."""
    M, g = 512, 64
    inp = W.make_inputs(W.Problem(name, M, N, K, W.INT4, g, 126, 0 if N > K else 1, affine=True), seed=0)
    y, _ = _run(inp, g)
    rows = np.array(sorted(set(range(24)) | set(range(M - 24, M)) | {63, 64, 191, 192, 287, 288, 383, 384}))
    _check(y, inp, g, name, rows=rows)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(y)))


def test_edge_cases():
    t = torch()
    inp = W.make_inputs(_problem(8, 32, 128, 64, cid=127), seed=7)
    words, _ = lb.pack_u4(_dev_levels(inp.codes))
    x, s, b = dev_x(inp.x), dev_scales(inp.scales), dev_scales(inp.biases)
    # M = 0: nothing to do
    y0 = lb.gemm_affine(t.zeros((0, 128), dtype=t.bfloat16, device="cuda"), words, s, b, 64)
    assert tuple(y0.shape) == (0, 32)
    # K = 0: an empty sum
    yk = t.full((5, 32), 3.0, dtype=t.bfloat16, device="cuda")
    lb.gemm_affine(t.zeros((5, 0), dtype=t.bfloat16, device="cuda"), t.zeros((32, 0), dtype=t.int32, device="cuda"),
                   t.zeros((32, 0), dtype=t.float16, device="cuda"), t.zeros((32, 0), dtype=t.float16, device="cuda"),
                   64, out=yk)
    t.cuda.synchronize()
    assert not yk.float().abs().sum().item()
    # g = 32 is not supported for 4-bit levels; a null bias pointer is refused
    with pytest.raises(lb.LowbitError) as e:
        lb.gemm_affine(x, words, dev_scales(np.ones((32, 4), np.float16)), dev_scales(np.ones((32, 4), np.float16)), 32)
    assert e.value.status == 2
    L = lb.lib()
    y = t.empty((8, 32), dtype=t.bfloat16, device="cuda")
    st = L.lowbit_gemm_affine(x.data_ptr(), words.data_ptr(), s.data_ptr(), None, y.data_ptr(), 8, 32, 128, 64, None)
    assert st == 1
    # the empty pack
    w0, bad = lb.pack_u4(t.zeros((0, 64), dtype=t.uint8, device="cuda"))
    assert bad == 0 and tuple(w0.shape) == (0, 8)


@pytest.mark.parametrize("M,N,K,g", [(512, 2560, 9728, 64), (64, 1024, 1536, 64), (100, 1040, 3072, 128),
                                     (37, 400, 2944, 64)])
def test_split_k_through_workspace(M, N, K, g):
    """lowbit_gemm_affine_ex: K split across three workgroups per tile where the 64 x 128 grid leaves
    compute units idle (the text encoder's down projection, smaller grids, ragged M and N, uneven
    K ranges), against the oracle; bitwise the same on a second call with the same workspace, whose
    arrival counters are back at zero after each call."""
    t = torch()
    need = lb.affine_workspace_size(M, N, K, g)
    assert need > 4096, (M, N, K, g, need)
    inp = W.make_inputs(_problem(M, N, K, g, cid=129), seed=9)
    words, _ = lb.pack_u4(_dev_levels(inp.codes))
    x, s, b = dev_x(inp.x), dev_scales(inp.scales), dev_scales(inp.biases)
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    y1 = host_bits(lb.gemm_affine(x, words, s, b, g, workspace=ws))
    assert not ws[:4096].any().item(), "arrival counters not reset"
    y2 = host_bits(lb.gemm_affine(x, words, s, b, g, workspace=ws))
    assert np.array_equal(y1, y2), "split-K result not deterministic"
    rows = None if M <= 128 else np.array(sorted(set(range(24)) | set(range(M - 24, M)) | {63, 64, 127, 128, 255, 256}))
    _check(y1, inp, g, f"split K {M}x{N}x{K} g{g}", rows=rows)
    # too small a workspace: exactly the unsplit call
    small = t.zeros(need - 16, dtype=t.uint8, device="cuda")
    y0 = host_bits(lb.gemm_affine(x, words, s, b, g))
    assert np.array_equal(host_bits(lb.gemm_affine(x, words, s, b, g, workspace=small)), y0)


def test_split_k_sizes():
    # shapes whose grid fills the machine, or with too few steps, take no split
    assert lb.affine_workspace_size(512, 19456, 2560, 64) == 0
    assert lb.affine_workspace_size(4096, 2560, 9728, 64) == 0
    assert lb.affine_workspace_size(64, 1024, 1024, 64) == 0
    assert lb.affine_workspace_size(512, 2560, 9728, 32) == 0
