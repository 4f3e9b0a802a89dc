"""GPU parity of the resident kernel's split along K across workgroups (skinny ternary
problems through a caller workspace: lowbit_gemm_ex, lowbit_gemm_batched_ex), against the
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
# the arrival counters of a split launch: the workspace's first 4 KiB, whatever the shape
COUNTER_BYTES = 4096


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _inputs(M, N, K, g, seed=0, cid=80):
    p = W.Problem("split", M, N, K, 2, g, cid, (M * 7 + N * 3 + K + g) % 100000)
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


def _workspace(n):
    t = torch()
    return t.zeros(max(n, 16), dtype=t.uint8, device="cuda")


# (N, K): K too long for the whole-K plan (the activations exceed the LDS); even and uneven
# K ranges; whole and partial column groups; few and many column blocks
@pytest.mark.parametrize("N,K", [(512, 6144), (3072, 9216), (3072, 12288), (1040, 8192), (256, 5120),
                                 (2048, 16384), (4112, 6144)])
@pytest.mark.parametrize("g", [64, 128])
def test_split_through_workspace(N, K, g):
    M = 16
    n = lb.workspace_size(M, N, K, g, 2)
    assert n > 0, (N, K)
    inp = _inputs(M, N, K, g, seed=1)
    x, w, s = _dev(inp)
    ws = _workspace(n)
    y1 = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
    _check(y1, inp, g, f"split N={N} K={K} g={g}")
    # the call leaves the counters at zero: the same workspace gives bitwise the same result
    y2 = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
    torch().cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert not ws[:COUNTER_BYTES].any().item(), "arrival counters not reset"


@pytest.mark.parametrize("M", [1, 3, 8, 15])
def test_split_rows(M):
    N, K = 3072, 12288
    inp = _inputs(M, N, K, 64, seed=2)
    x, w, s = _dev(inp)
    ws = _workspace(lb.workspace_size(M, N, K, 64, 2))
    y = host_bits(lb.gemm(x, w, s, 64, 2, workspace=ws))
    _check(y, inp, 64, f"split M={M}")


def test_one_workspace_for_every_shape():
    # one workspace, sized for the largest need, serves calls of different shapes in turn
    shapes = [(3072, 12288), (512, 6144), (3072, 9216), (3072, 3072)]
    ws = _workspace(max(lb.workspace_size(16, N, K, 64, 2) for N, K in shapes))
    for i, (N, K) in enumerate(shapes * 2):
        inp = _inputs(16, N, K, 64, seed=3 + i % 4)
        x, w, s = _dev(inp)
        y = host_bits(lb.gemm(x, w, s, 64, 2, workspace=ws))
        _check(y, inp, 64, f"shared workspace {N}x{K}")
    assert not ws[:COUNTER_BYTES].any().item()


def test_batched_pairs_through_workspace():
    # the image and text stream linears of a double-stream block at M = 16, as one batched
    # call with a workspace: the K-heavy pair is split, the others run whole
    t = torch()
    for (N, K) in [(3072, 9216), (9216, 3072), (3072, 3072)]:
        inps = [_inputs(16, N, K, 64, seed=9 + i, cid=81) for i in range(2)]
        probs = []
        for inp in inps:
            x, w, s = _dev(inp)
            probs.append((x, w, s, t.empty((16, N), dtype=t.bfloat16, device="cuda"), 64, 2))
        n = lb.batched_workspace_size(probs)
        ws = _workspace(n)
        lb.gemm_batched(probs, workspace=ws)
        t.cuda.synchronize()
        first = [host_bits(p[3]).copy() for p in probs]
        lb.gemm_batched(probs, workspace=ws)
        t.cuda.synchronize()
        for i, inp in enumerate(inps):
            assert np.array_equal(first[i], host_bits(probs[i][3])), f"{N}x{K} problem {i} not deterministic"
            _check(first[i], inp, 64, f"batched {N}x{K} problem {i} ws={n}")
        assert not ws[:COUNTER_BYTES].any().item()


def test_ex_falls_back_without_enough_workspace():
    t = torch()
    M, N, K = 16, 512, 6144
    inp = _inputs(M, N, K, 64, seed=5)
    x, w, s = _dev(inp)
    plain = host_bits(lb.gemm(x, w, s, 64, 2))
    small = t.zeros(64, dtype=t.uint8, device="cuda")
    assert np.array_equal(host_bits(lb.gemm(x, w, s, 64, 2, workspace=small)), plain)
    # shapes the split does not take need no workspace and equal lowbit_gemm
    for (MM, g, bits) in ((32, 64, 2), (16, 64, 1), (16, 32, 2)):
        assert lb.workspace_size(MM, N, K, g, bits) == 0
        p = W.Problem("fb", MM, N, K, bits, g, 82, MM + g + bits)
        inp2 = W.make_inputs(p, 6)
        x2 = dev_x(inp2.x)
        w2, _ = lb.pack(dev_codes(inp2.codes), bits)
        s2 = dev_scales(inp2.scales)
        a = host_bits(lb.gemm(x2, w2, s2, g, bits))
        b = host_bits(lb.gemm(x2, w2, s2, g, bits, workspace=small))
        assert np.array_equal(a, b)


def test_split_one_hot_bit_exact():
    # one nonzero code: only one K range has a nonzero partial sum, so the split result is
    # exactly RNE_bf16(c * s * x)
    M, N, K, g = 16, 3072, 12288, 64
    x = W.gen_x(W.rng_for(4, 83, 0), M, K)
    s = W.gen_scales(W.rng_for(4, 83, 1), N, K, g)
    xf = oracle.bf16_bits_to_f64(x)
    ws = _workspace(lb.workspace_size(M, N, K, g, 2))
    xd, sd = dev_x(x), dev_scales(s)
    for (n0, k0, c0) in ((0, 0, 1), (191, 767, -1), (192, 768, 1), (3071, 12287, -1), (1300, 5000, 1)):
        c = np.zeros((N, K), dtype=np.int8)
        c[n0, k0] = c0
        w, _ = lb.pack(dev_codes(c), 2)
        y = host_bits(lb.gemm(xd, w, sd, g, 2, workspace=ws))
        want = oracle.f64_to_bf16_bits_rne(c0 * float(s[n0, k0 // g]) * xf[:, k0])
        col = y[:, n0]
        zero = lambda b: (b & 0x7FFF) == 0
        assert ((col == want) | (zero(col) & zero(want))).all(), (n0, k0)
        assert np.all(zero(np.delete(y, n0, axis=1)))


def test_default_choice_large_n_whole_k():
    # N = 27648 fills the machine without splitting K: lowbit_gemm picks the resident kernel
    # whole, and needs no workspace
    assert lb.variant(16, 27648, 3072, 64, 2) == "resident"
    assert lb.workspace_size(16, 27648, 3072, 64, 2) == 0
    inp = _inputs(16, 27648, 3072, 64, seed=7)
    y1, _ = run_gemm(inp, 64, 2)
    y2, _ = run_gemm(inp, 64, 2)
    assert np.array_equal(y1, y2)
    cols = np.random.default_rng(0).choice(27648, 2048, replace=False)
    _check(y1[:, cols], W.Inputs(inp.x, inp.codes[cols], inp.scales[cols]), 64, "N=27648 sampled columns")


def test_workspace_shared_by_launches_of_different_tile_counts():
    """One workspace serves a split launch with few column groups (16x3072x12288: 32 tiles),
    then launches with many (16x18432x6144: 128 tiles), as single calls and as a batched call
    that mixes both K.  The first launch leaves its fp32 partial sums in the workspace; every
    later launch must still find its arrival counters at zero and every result must meet the
    oracle."""
    t = torch()
    small, large = (3072, 12288), (18432, 6144)
    need = max(lb.workspace_size(16, N, K, 64, 2) for N, K in (small, large))
    items = []
    for i, (N, K) in enumerate((small, large, small, large)):
        inp = _inputs(16, N, K, 64, seed=20 + i, cid=84)
        x, w, s = _dev(inp)
        items.append((inp, (x, w, s, t.empty((16, N), dtype=t.bfloat16, device="cuda"), 64, 2)))
    need = max(need, lb.batched_workspace_size([a for _, a in items]))
    ws = _workspace(need)
    for rep in range(2):
        for inp, (x, w, s, y, g, bits) in items[:2]:
            yb = host_bits(lb.gemm(x, w, s, g, bits, workspace=ws))
            _check(yb, inp, g, f"shared workspace {tuple(x.shape)}x{w.shape[0]} pass {rep}")
            assert not ws[:COUNTER_BYTES].any().item(), "arrival counters not reset"
    lb.gemm_batched([a for _, a in items], workspace=ws)
    t.cuda.synchronize()
    for inp, (x, w, s, y, g, bits) in items:
        _check(host_bits(y), inp, g, f"batched, shared workspace {tuple(x.shape)}x{w.shape[0]}")
    assert not ws[:COUNTER_BYTES].any().item(), "arrival counters not reset"


def test_concurrent_streams_with_their_own_workspaces():
    """Two streams, each with its own workspace, run split-K calls at the same time: every result
    is bitwise its single-stream result and both counter regions end at zero."""
    t = torch()
    M, g = 16, 64
    data = []
    for i, (N, K) in enumerate(((3072, 12288), (3072, 9216))):
        inp = _inputs(M, N, K, g, seed=20 + i, cid=90 + i)
        x, w, s = _dev(inp)
        ws = _workspace(lb.workspace_size(M, N, K, g, 2))
        ref = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
        _check(ref, inp, g, f"split N={N} K={K}")
        data.append((x, w, s, ws, ref, t.empty((M, N), dtype=t.bfloat16, device="cuda")))
    streams = [t.cuda.Stream(), t.cuda.Stream()]  # default priority
    for st in streams:
        st.wait_stream(t.cuda.current_stream())
    outs = [[], []]
    for _ in range(20):
        for (x, w, s, ws, _ref, y), st, o in zip(data, streams, outs):
            with t.cuda.stream(st):
                lb.gemm(x, w, s, g, 2, out=y, workspace=ws)
                o.append(y.clone())
    for st in streams:
        t.cuda.current_stream().wait_stream(st)
    t.cuda.synchronize()
    for (_x, _w, _s, ws, ref, _y), o in zip(data, outs):
        for y in o:
            assert np.array_equal(host_bits(y), ref)
        assert not ws[:COUNTER_BYTES].any().item(), "arrival counters not reset"
