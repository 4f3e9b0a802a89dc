"""GPU parity of stream-K on the 256 x 256 tile (LOWBIT_VARIANT=tile256sk through a workspace):
every workgroup takes a contiguous range of the (tile, 64-element step) units, and tiles split
between workgroups are summed from fp32 partial tiles.  Checked against the oracle on shapes whose
tiles have one part, two parts (the finisher adds the other part in its epilogue) and three or more
(every part through the workspace), with ragged edges, the g = 32 K tail and binary codes; every
call is repeated for bitwise determinism and leaves the arrival counters at zero."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3
COUNTER_BYTES = 4096  # the workspace's arrival counters
BM = BN = 256
KS = 64


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def _parts_per_tile(M, N, K):
    """Most workgroups that share one tile under the kernel's partition."""
    tiles = -(-M // BM) * -(-N // BN)
    ks = -(-K // KS)
    U = tiles * ks
    nwg = min(256, U)
    owner = [((u + 1) * nwg - 1) // U for u in range(U)]
    return max(owner[t * ks + ks - 1] - owner[t * ks] + 1 for t in range(tiles))


def _setup(M, N, K, g, bits, seed):
    inp = W.make_inputs(W.Problem("streamk", M, N, K, bits, g, 170, (M * 3 + N * 5 + K + g) % 99991), seed)
    w, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    return inp, dev_x(inp.x), w, dev_scales(inp.scales)


def _check(y, inp, g, rows, what):
    sel = np.arange(y.shape[0]) if rows is None else np.array(rows)
    r = oracle.check_tolerance(y[sel], oracle.gemm_ref_f64(inp.x[sel], inp.codes, inp.scales, g))
    assert r["ok"], f"{what}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']}"


def _workspace(n):
    t = torch()
    return t.zeros(max(n, 16), dtype=t.uint8, device="cuda")


@pytest.mark.parametrize("M,N,K,g,bits,rows,parts", [
    (200, 304, 64, 64, 2, None, 1),                              # 2 units on 2 workgroups: whole tiles only
    (256, 256, 640, 64, 2, None, 10),                            # one tile over 10 workgroups
    (300, 528, 3072, 64, 2, None, 43),                           # 6 tiles over 256 workgroups, ragged M and N
    (4352, 4096, 256, 64, 2, (0, 255, 256, 2176, 4095, 4096, 4351), 2),   # 272 tiles: two parts at most
    (4608, 9216, 256, 64, 2, (0, 1, 2303, 2304, 4607), 2),       # ranges of whole tiles and two parts
    (4608, 3072, 512, 64, 2, (0, 511, 512, 3000, 4607), 3),      # 216 tiles: two and three parts
    (1000, 1008, 4128, 32, 2, (0, 255, 256, 767, 768, 999), 16),  # g = 32, K % 64 == 32 (a half step)
    (2304, 2560, 1152, 128, 1, (0, 767, 768, 2303), 4),          # binary g = 128
    (777, 1232, 2048, 64, 1, None, 14),                          # binary g = 64, ragged M and N
])
def test_streamk_parity(M, N, K, g, bits, rows, parts, monkeypatch, capfd):
    assert _parts_per_tile(M, N, K) == parts
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256sk")
    n = lb.workspace_size(M, N, K, g, bits)
    nwg = min(256, -(-M // BM) * -(-N // BN) * -(-K // KS))
    assert n == COUNTER_BYTES + 2 * nwg * BM * BN * 4, n
    print(f"stream-K {M}x{N}x{K} g={g} bits={bits} parts<={parts}", flush=True)
    inp, x, w, s = _setup(M, N, K, g, bits, seed=1)
    ws = _workspace(n)
    monkeypatch.setenv("LOWBIT_TRACE", "1")
    y1 = host_bits(lb.gemm(x, w, s, g, bits, workspace=ws))
    monkeypatch.delenv("LOWBIT_TRACE")
    assert "streamk" in capfd.readouterr().err, "the stream-K kernel did not run"
    _check(y1, inp, g, rows, f"stream-K {M}x{N}x{K} g={g} bits={bits}")
    assert not ws[:COUNTER_BYTES].any().item(), "arrival counters not reset"
    # a second call on the same workspace: bitwise the same (the sums run in one fixed order)
    for _ in range(2):
        y2 = host_bits(lb.gemm(x, w, s, g, bits, workspace=ws))
        assert np.array_equal(y1, y2), "stream-K result changed between calls"
    assert not ws[:COUNTER_BYTES].any().item()


def test_streamk_short_workspace_runs_the_plain_tile(monkeypatch):
    # a workspace too small for the partial tiles: the call runs the 256 x 256 tile without a split
    M, N, K, g = 1024, 768, 1024, 64
    inp, x, w, s = _setup(M, N, K, g, 2, seed=2)
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256w")
    y_plain = host_bits(lb.gemm(x, w, s, g, 2))
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256sk")
    ws = _workspace(lb.workspace_size(M, N, K, g, 2) - 16)
    y = host_bits(lb.gemm(x, w, s, g, 2, workspace=ws))
    assert np.array_equal(y, y_plain)
    assert lb.variant(M, N, K, g, 2) == "tile256x256"


def test_streamk_batched_and_shared_with_the_resident_split(monkeypatch):
    # one workspace serves a resident split call (M = 16, its counters in the same first 4 KiB),
    # a batched stream-K call of two problems, and the resident call again
    t = torch()
    ws = _workspace(max(lb.workspace_size(16, 3072, 12288, 64, 2),
                        COUNTER_BYTES + 2 * 256 * BM * BN * 4))
    inp16, x16, w16, s16 = _setup(16, 3072, 12288, 64, 2, seed=3)
    y16 = host_bits(lb.gemm(x16, w16, s16, 64, 2, workspace=ws))
    _check(y16, inp16, 64, None, "resident split before")
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256sk")
    probs, inps = [], []
    for i, (M, N, K) in enumerate([(1536, 3072, 1024), (512, 2048, 3072)]):
        inp, x, w, s = _setup(M, N, K, 64, 2, seed=10 + i)
        inps.append(inp)
        probs.append((x, w, s, t.empty((M, N), dtype=t.bfloat16, device="cuda"), 64, 2))
    assert lb.batched_workspace_size(probs) <= ws.numel()
    lb.gemm_batched(probs, workspace=ws)
    for inp, pr in zip(inps, probs):
        _check(host_bits(pr[3]), inp, 64, (0, 255, 256, inp.x.shape[0] - 1), "batched stream-K")
    assert not ws[:COUNTER_BYTES].any().item()
    monkeypatch.delenv("LOWBIT_VARIANT")
    y16b = host_bits(lb.gemm(x16, w16, s16, 64, 2, workspace=ws))
    assert np.array_equal(y16, y16b)
    assert not ws[:COUNTER_BYTES].any().item()


@pytest.mark.parametrize("M,N,K,g,bits,rows", [
    (1536, 18432, 3072, 64, 2, (0, 255, 256, 767, 1279, 1280, 1535)),   # 1.69 rounds of 256 x 256 tiles
    (4608, 9216, 3072, 128, 1, (0, 1, 2303, 2304, 4351, 4352, 4607)),   # binary g = 128: 2.53 rounds
])
def test_streamk_at_full_size(M, N, K, g, bits, rows, monkeypatch, capfd):
    # the denoise-step shapes where stream-K beats every whole-tile launch when timed alone: with
    # a workspace the call runs stream-K; the allocation-free entry point and the call without a
    # workspace run the 256 x 256 tile whole, and both agree with the oracle
    monkeypatch.setenv("LOWBIT_VARIANT", "tile256sk")
    n = lb.workspace_size(M, N, K, g, bits)
    assert n == COUNTER_BYTES + 2 * 256 * BM * BN * 4
    print(f"stream-K {M}x{N}x{K} g={g} bits={bits}", flush=True)
    inp, x, w, s = _setup(M, N, K, g, bits, seed=4)
    ws = _workspace(n)
    capfd.readouterr()
    monkeypatch.setenv("LOWBIT_TRACE", "1")
    y_sk = host_bits(lb.gemm(x, w, s, g, bits, workspace=ws))
    y_plain = host_bits(lb.gemm(x, w, s, g, bits))
    t = torch()
    out = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    y_na = host_bits(lb.gemm_noalloc(x, w, s, g, bits, out))
    monkeypatch.delenv("LOWBIT_TRACE")
    log = [l for l in capfd.readouterr().err.splitlines() if l.startswith("lowbit: ")]
    assert len(log) == 3 and "streamk" in log[0] and "streamk" not in log[1] + log[2], log
    assert np.array_equal(y_plain, y_na)
    for y, what in ((y_sk, "stream-K"), (y_plain, "whole tiles")):
        _check(y, inp, g, rows, f"{what} {M}x{N}x{K} g={g} bits={bits}")
    assert not ws[:COUNTER_BYTES].any().item()
