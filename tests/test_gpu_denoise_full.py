"""GPU parity of one FLUX.2 Klein 4B denoise step at 1024x1024 at its real sizes (the 80-GEMM
sweep, ternary g = 64): every distinct linear of the step against the oracle, on all output
columns of sampled rows -- the first and last rows, the rows either side of every 256- and
288-row tile boundary, and random rows.

* the single-stream blocks' fused 3072 -> 27648 linear and their 12288 -> 3072 output linear at
  M = 4608 (4096 image + 512 text tokens, concatenated);
* the double-stream blocks' image-stream linears at M = 4096 (QKV, proj, MLP-in, MLP-out) as
  single calls;
* each image / text pair ({4096, 512} rows, separate weights) as one grouped call, with and
  without a workspace, and -- with the tile fixed -- bitwise equal to single calls on that tile.

Shapes: the model card "bonsai-image-binary-4B-gemlite-1bit", section "Model Overview" (5
double-stream + 20 single-stream blocks, every matmul-heavy linear quantised); token counts
(H/16)(W/16) image + 512 text tokens (mlx-vlm Prism Bonsai guide, section 组件架构)."""
from __future__ import annotations

import numpy as np
import pytest

import binary_bit_gemm_amd as lb
import oracle
import workloads as W
from tests.gpu_helpers import dev_codes, dev_scales, dev_x, host_bits, torch

pytestmark = pytest.mark.gpu

REL_ALARM = 2.5e-3
SWEEP = W.denoise_step_sweep()
BY_NAME = {p.name: p for p in SWEEP}
KINDS = ["qkv", "proj", "mlp_in", "mlp_out"]


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    assert lb.lib().lowbit_device_supported(0) == 1, "device 0 is not gfx950"
    yield


def sample_rows(M: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(range(min(M, 24))) | set(range(max(0, M - 24), M))
    for tile in (256, 288):
        for b in range(tile, M, tile):
            rows |= {b - 1, b}
    rows |= set(rng.choice(M, size=min(M, 32), replace=False).tolist())
    return np.array(sorted(rows))


def check_rows(y_bits, inp, g, rows, what):
    yref = oracle.gemm_ref_f64(inp.x[rows], inp.codes, inp.scales, g)
    r = oracle.check_tolerance(y_bits[rows], yref)
    assert r["ok"], f"{what}: {r}"
    assert r["rel_frob"] <= REL_ALARM, f"{what}: rel_frob {r['rel_frob']} above alarm"


def device_problem(p: W.Problem, seed: int = 0):
    t = torch()
    inp = W.make_inputs(p, seed)
    x = dev_x(inp.x)
    w, bad = lb.pack(dev_codes(inp.codes), p.bits)
    assert bad == 0
    s = dev_scales(inp.scales)
    y = t.full((p.M, p.N), float("nan"), dtype=t.bfloat16, device="cuda")
    return inp, (x, w, s, y, p.g, p.bits)


@pytest.mark.parametrize("name", ["s0_fused", "s0_out"])
def test_single_stream_linears_full_size(name):
    p = BY_NAME[name]
    assert p.M == 4608
    inp, (x, w, s, y, g, bits) = device_problem(p)
    lb.gemm(x, w, s, g, bits, out=y)
    torch().cuda.synchronize()
    yb = host_bits(y)
    check_rows(yb, inp, g, sample_rows(p.M, p.tensor_id), f"{name} {p.M}x{p.N}x{p.K}")
    # every row written (no NaN left from the fill), and the spread matches
    # Var(y) = K * P(c != 0) * E[s^2] with E[s^2] = 9.25e-4 for U[0.005, 0.05]
    yf = oracle.bf16_bits_to_f64(yb)
    assert np.all(np.isfinite(yf))
    assert abs(yf.var() / (p.K * 0.5 * 9.25e-4) - 1) < 0.05


@pytest.mark.parametrize("kind", KINDS)
def test_image_stream_linear_full_size(kind):
    p = BY_NAME[f"d0_img_{kind}"]
    assert p.M == 4096
    inp, (x, w, s, y, g, bits) = device_problem(p)
    lb.gemm(x, w, s, g, bits, out=y)
    torch().cuda.synchronize()
    yb = host_bits(y)
    check_rows(yb, inp, g, sample_rows(p.M, p.tensor_id), f"{p.name} {p.M}x{p.N}x{p.K}")
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(yb)))


@pytest.mark.parametrize("kind", KINDS)
def test_image_text_pair_grouped_full_size(kind, monkeypatch):
    t = torch()
    img, txt = BY_NAME[f"d0_img_{kind}"], BY_NAME[f"d0_txt_{kind}"]
    assert (img.M, txt.M) == (4096, 512) and (img.N, img.K) == (txt.N, txt.K)
    items = [device_problem(img), device_problem(txt)]
    probs = [a for _, a in items]
    rows = [sample_rows(img.M, img.tensor_id), sample_rows(txt.M, txt.tensor_id)]

    lb.gemm_batched(probs)
    t.cuda.synchronize()
    grouped = [host_bits(a[3]).copy() for a in probs]
    for (inp, a), yb, rr, p in zip(items, grouped, rows, (img, txt)):
        check_rows(yb, inp, a[4], rr, f"grouped {p.name}")

    # through lowbit_gemm_batched_ex: at these row counts no launch splits K, so the workspace
    # changes nothing
    ws = t.zeros(max(16, lb.batched_workspace_size(probs)), dtype=t.uint8, device="cuda")
    for a in probs:
        a[3].fill_(float("nan"))
    lb.gemm_batched(probs, workspace=ws)
    t.cuda.synchronize()
    for a, want in zip(probs, grouped):
        assert np.array_equal(host_bits(a[3]), want), "batched_ex differs from batched"

    # with the tile fixed for both, a problem's bits do not depend on the other problem of
    # the launch: the grouped result equals the single calls'
    for v in ("tile288", "tile256w"):
        monkeypatch.setenv("LOWBIT_VARIANT", v)
        singles = [host_bits(lb.gemm(x, w, s, g, bits)) for (x, w, s, y, g, bits) in probs]
        for a in probs:
            a[3].fill_(float("nan"))
        lb.gemm_batched(probs)
        t.cuda.synchronize()
        for a, single, p in zip(probs, singles, (img, txt)):
            assert np.array_equal(host_bits(a[3]), single), f"{v}: grouped {p.name} differs from its single call"
    monkeypatch.delenv("LOWBIT_VARIANT")
