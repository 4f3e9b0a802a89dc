"""Sanity of the seeded input generators (CPU only)."""
import numpy as np

import workloads as W


def test_x_is_bf16_rne_of_normal():
    import torch
    rng = W.rng_for(0, 1, 0)
    x = W.gen_x(rng, 64, 512)
    ref = W.rng_for(0, 1, 0).standard_normal((64, 512), dtype=np.float32)
    t = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(x, t)


def test_code_distributions():
    c = W.gen_codes(W.rng_for(0, 1, 1), 512, 1024, W.TERNARY)
    frac = [(c == v).mean() for v in (-1, 0, 1)]
    assert abs(frac[0] - 0.25) < 0.01 and abs(frac[1] - 0.5) < 0.01 and abs(frac[2] - 0.25) < 0.01
    b = W.gen_codes(W.rng_for(0, 2, 1), 512, 1024, W.BINARY)
    assert set(np.unique(b)) == {-1, 1} and abs((b == 1).mean() - 0.5) < 0.01


def test_scales_range():
    s = W.gen_scales(W.rng_for(0, 1, 2), 256, 3072, 64)
    assert s.dtype == np.float16 and s.shape == (256, 48)
    assert s.min() >= np.float16(0.005) and s.max() <= np.float16(0.05)


def test_seeded_and_distinct():
    p = W.Problem("a", 8, 32, 128)
    a, b = W.make_inputs(p), W.make_inputs(p)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.codes, b.codes)
    q = W.Problem("b", 8, 32, 128, tensor_id=1)
    assert not np.array_equal(W.make_inputs(q).codes, a.codes)


def test_denoise_step_sweep_shape_count():
    probs = W.denoise_step_sweep()
    assert len(probs) == 80
    flops = sum(p.flops for p in probs)
    assert abs(flops / 1e12 - 28.27) < 0.01
    skinny = W.denoise_step_sweep(skinny_m=16)
    assert all(p.M == 16 for p in skinny) and len(skinny) == 80


def test_bench_reads_kernel_variants_from_the_launch_log():
    """bench.py names the kernels a step launches from the library's LOWBIT_TRACE lines: tile
    families by their tile (the 16x16-block kernel's K split as a k2 suffix), the skinny-M
    kernels by family; other lines are ignored."""
    import bench
    lines = {
        "lowbit: tile16 288x192 waves=2x6x1 epi=plain g=64 bits=2 grid=256 block=768 lds=0 problems=4608x3072x3072":
            "tile288x192",
        "lowbit: tile16 96x192 waves=1x4x2 epi=plain g=64 bits=2 grid=256 block=512 lds=0 problems=1536x3072x3072":
            "tile96x192k2",
        "lowbit: tile16 96x192 waves=1x4x1 epi=plain g=64 bits=2 grid=256 block=256 lds=0 problems=1536x3072x3136":
            "tile96x192",
        "lowbit: tile16 64x128 waves=1x4x1 epi=plain affine g=64 bits=4 grid=160 block=256 lds=0 problems=512x2560x9664":
            "tile64x128k2",
        "lowbit: tile16 256x192 waves=2x6x1 epi=plain g=64 bits=2 grid=256 block=768 lds=0 problems=4096x3072x3072":
            "tile256x192",
        "lowbit: tiled32 256x256 waves=2x4 g=128 bits=1 grid=216 block=512 lds=0 problems=4608x3072x3072":
            "tile256x256",
        "lowbit: tiled32 256x256 waves=2x4 streamk g=128 bits=1 grid=256 block=512 lds=0 problems=4608x9216x3072":
            "tile256x256sk",
        "lowbit: resident column_blocks=7 k_slices=2 steps=6 splits=1 tiles=247 epi=plain g=64 bits=2 grid=247 "
        "block=896 lds=110000 problems=16x27648x3072": "resident",
        "lowbit: skinny row_blocks=1 column_blocks=1 waves=4 g=64 bits=2 grid=384 block=256 lds=0 "
        "problems=16x3072x3072,16x3072x3072": "skinny",
        "/opt/amdgpu/share/libdrm/amdgpu.ids: No such file or directory": None,
    }
    for line, want in lines.items():
        assert bench.variant_of_trace_line(line) == want, line
    # every name it can produce is one the traffic hash knows the sources of
    for want in lines.values():
        assert want is None or want in bench.VARIANT_SOURCES, want
