"""Re-derive the tile model's per-tile efficiencies from measurements on the GPU.

    python -m binary_bit_gemm_amd.tune_tiles [--bits 2] [--g 64] [--reps 30] [--shapes M,N,K ...]

The tile choice (gemm_tiled.hip, pick_tile_variant) costs a tile variant t on a shape as

    cost(t) = rounds(t) * per_cu(t) * BM(t) * BN(t) / eff(t),
    rounds(t) = ceil(tiles(t) / (256 compute units * per_cu(t)))

and picks the cheapest.  eff(t) is the tile's work per unit time relative to the 256 x 256 tile.
This script times every tile variant (forced with LOWBIT_VARIANT) on each shape with HIP events
around back-to-back calls, and prints for each (shape, tile) the time, the TFLOP/s and the implied
efficiency

    eff(t) = [rounds(t) * per_cu(t) * BM * BN / time(t)] / [the same for 256 x 256],

i.e. the value of eff(t) that makes the cost model reproduce the measured time ratio on that
shape.  Its median over shapes is the constant to put in the table.  Inputs are seeded random
ternary (or binary / 4-bit) weights; the library's kernels run unchanged.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# name for LOWBIT_VARIANT -> (tile rows, tile columns, workgroups resident per compute unit)
TILES = {
    "tile256w": (256, 256, 1), "tile288": (288, 192, 1), "tile256n": (256, 192, 1), "tile128": (128, 256, 2),
    "tile64": (64, 256, 2),
    "tile96": (96, 192, 1), "tile96k2": (96, 192, 1), "tile64k2": (64, 128, 1),
    "tile256sk": (256, 256, 1),  # stream-K: the work spread evenly over every compute unit
}
STREAM_K = {"tile256sk"}
DEFAULT_SHAPES = [(4608, 3072, 3072), (4608, 9216, 3072), (4608, 18432, 3072), (4608, 3072, 9216),
                  (4608, 3072, 12288), (4096, 4096, 3072), (4096, 3072, 3072), (4096, 9216, 3072),
                  (1536, 3072, 3072), (1536, 9216, 3072)]
CUS = 256


def inputs(M, N, K, g, bits, seed=0):
    import torch
    import binary_bit_gemm_amd as lb
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + M * 7 + N * 3 + K)
    x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    if bits == 2:
        lut = torch.tensor([-1, 0, 0, 1], dtype=torch.int8, device="cuda")
        codes = lut[torch.randint(0, 4, (N, K), generator=gen, device="cuda")]
    elif bits == 1:
        codes = torch.randint(0, 2, (N, K), generator=gen, device="cuda", dtype=torch.int8) * 2 - 1
    else:
        codes = torch.randint(-8, 8, (N, K), generator=gen, device="cuda", dtype=torch.int8)
    w, _ = lb.pack(codes.contiguous(), bits, count_invalid=False)
    s = (torch.rand((N, K // g), generator=gen, device="cuda") * 0.045 + 0.005).to(torch.float16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    return x, w, s, y


def time_us(fn, reps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def weighted_work(tile, M, N):
    bm, bn, per_cu = TILES[tile]
    tiles = math.ceil(M / bm) * math.ceil(N / bn)
    rounds = tiles / (CUS * per_cu) if tile in STREAM_K else math.ceil(tiles / (CUS * per_cu))
    return rounds * per_cu * bm * bn


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--bits", type=int, default=2)
    ap.add_argument("--g", type=int, default=64)
    ap.add_argument("--reps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--tiles", default="tile256w,tile288,tile256n,tile128,tile64,tile96,tile96k2")
    ap.add_argument("--shapes", nargs="*", default=None, help="M,N,K triples")
    a = ap.parse_args()
    import binary_bit_gemm_amd as lb
    shapes = [tuple(int(v) for v in s.split(",")) for s in a.shapes] if a.shapes else DEFAULT_SHAPES
    tiles = [t for t in a.tiles.split(",") if t]
    effs = {t: [] for t in tiles}
    for (M, N, K) in shapes:
        x, w, s, y = inputs(M, N, K, a.g, a.bits)
        row = {}
        for t in tiles:
            os.environ["LOWBIT_VARIANT"] = t
            if t in ("tile96k2", "tile64k2") and (K // 64) % 2:
                continue
            ws = None
            if t in STREAM_K:  # partial tiles through a workspace
                import torch
                ws = torch.zeros(lb.workspace_size(M, N, K, a.g, a.bits), dtype=torch.uint8, device="cuda")
            us = time_us(lambda: lb.gemm(x, w, s, a.g, a.bits, out=y, workspace=ws), a.reps, a.warmup)
            row[t] = us
            del ws
        os.environ.pop("LOWBIT_VARIANT", None)
        base = weighted_work("tile256w", M, N) / row["tile256w"] if "tile256w" in row else None
        for t, us in row.items():
            eff = (weighted_work(t, M, N) / us) / base if base else None
            if eff is not None:
                effs[t].append(eff)
            print(json.dumps({"shape": [M, N, K], "bits": a.bits, "g": a.g, "tile": t, "us": round(us, 2),
                              "tflops": round(2 * M * N * K / us / 1e6, 1),
                              "implied_eff": None if eff is None else round(eff, 3),
                              "auto": lb.variant(M, N, K, a.g, a.bits)}), flush=True)
    summary = {t: round(statistics.median(v), 3) for t, v in effs.items() if v}
    print(json.dumps({"median_implied_eff": summary, "bits": a.bits, "g": a.g}), flush=True)


if __name__ == "__main__":
    main()
