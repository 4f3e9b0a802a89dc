"""Times the M <= 16 kernels behind the planner's resident-kernel thresholds.

For each skinny shape (default: M = 16, the denoise step's N x K, plus N = 4096 / 6144 / 8192 at
K = 3072 around the 512-column-block threshold) this script times, with HIP events around 30
back-to-back calls after 10 warm-up calls, in 5 rounds that take the variants in turn (the median
per variant is printed: the first launches after a pause run slower):
  * skinny    -- the skinny kernel (LOWBIT_VARIANT=skinny),
  * resident  -- the resident kernel over the whole K (LOWBIT_VARIANT=resident, no workspace),
  * split     -- the resident kernel split along K through a workspace (the automatic plan of
                 lowbit_gemm_ex), where the planner makes one,
  * auto      -- the library's own choice without a workspace.
With --pair every call is a batched pair of two problems of the shape with their own weights (the
denoise step's image and text stream linears at M = 16), through lowbit_gemm_batched(_ex).
The calls rotate over copies of the weights (at least 512 MiB in total), so every call streams
its weights from HBM as the denoise step's distinct linears do, not from the 256 MiB Infinity
Cache.  Prints one JSON line per (shape, variant) and which variant the planner picks.

    python -m binary_bit_gemm_amd.tune_resident [--m 16] [--pair] [--shapes N,K ...]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_SHAPES = [(3072, 3072), (4096, 3072), (6144, 3072), (8192, 3072), (9216, 3072), (18432, 3072),
                  (27648, 3072), (3072, 9216), (3072, 12288)]
ROTATE_BYTES = 512 << 20


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, default=16)
    ap.add_argument("--g", type=int, default=64)
    ap.add_argument("--reps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--pair", action="store_true", help="batched pairs, as the denoise step runs them")
    ap.add_argument("--shapes", nargs="*", default=None, help="N,K pairs")
    a = ap.parse_args()
    import torch
    import binary_bit_gemm_amd as lb
    shapes = [tuple(int(v) for v in s.split(",")) for s in a.shapes] if a.shapes else DEFAULT_SHAPES
    M, g = a.m, a.g
    for (N, K) in shapes:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(M * 7 + N * 3 + K)
        x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
        lut = torch.tensor([-1, 0, 0, 1], dtype=torch.int8, device="cuda")
        codes = lut[torch.randint(0, 4, (N, K), generator=gen, device="cuda")]
        w0, _ = lb.pack(codes.contiguous(), 2, count_invalid=False)
        del codes
        s = (torch.rand((N, K // g), generator=gen, device="cuda") * 0.045 + 0.005).to(torch.float16)
        copies = max(2, -(-ROTATE_BYTES // (w0.numel() * 4)))
        ws_list = [w0] + [w0.clone() for _ in range(copies - 1)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if a.pair:
            need = lb.batched_workspace_size([(x, w0, s, y, g, 2), (x, w0, s, y2, g, 2)])
        else:
            need = lb.workspace_size(M, N, K, g, 2)
        wsp = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")

        def timed(variant, workspace):
            if variant is None:
                os.environ.pop("LOWBIT_VARIANT", None)
            else:
                os.environ["LOWBIT_VARIANT"] = variant
            n = [0]

            def call():
                if a.pair:
                    wa, wb = ws_list[n[0] % copies], ws_list[(n[0] + 1) % copies]
                    lb.gemm_batched([(x, wa, s, y, g, 2), (x, wb, s, y2, g, 2)], workspace=workspace)
                    n[0] += 2
                else:
                    lb.gemm(x, ws_list[n[0] % copies], s, g, 2, out=y, workspace=workspace)
                    n[0] += 1
            for _ in range(a.warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(a.reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            os.environ.pop("LOWBIT_VARIANT", None)
            return e0.elapsed_time(e1) / a.reps * 1e3

        runs = {"skinny": ("skinny", None), "resident": ("resident", None), "auto": (None, None)}
        if need > 0:
            runs["split"] = (None, wsp)
        wbytes = (N * K // 4 + N * (K // g) * 2) * (2 if a.pair else 1)
        times = {name: [] for name in runs}
        for _ in range(a.rounds):
            for name, (variant, workspace) in runs.items():
                times[name].append(timed(variant, workspace))
        for name in runs:
            us = statistics.median(times[name])
            print(json.dumps({"M": M, "N": N, "K": K, "g": g, "pair": a.pair, "variant": name, "us": round(us, 2),
                              "GB/s": round(wbytes / us / 1e3, 1),
                              "auto_without_workspace": lb.variant(M, N, K, g, 2),
                              "workspace_bytes": need}), flush=True)
        del ws_list, w0, wsp
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
