"""Throughput of the packed low-bit weight GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload res1024|res512|res512_binary|sweep|skinny]

A step is one pass of the hot path over one batch of synthetic inputs that are already
resident in HBM: every GEMM of the workload, each with its own weights (the denoise-step
workloads launch a double-stream block's image and text linear of one kind as one grouped
call; --graph replays the step as one captured HIP graph).  Packing is the offline load-time step and
runs before the timed region.

Workloads (FLUX.2 Klein 4B MMDiT linears, hidden 3072):
  res1024        M = 4608 tokens (4096 image + 512 text) ternary g=64:
                 N x K = 3072x3072, 9216x3072, 18432x3072, 3072x9216, 3072x12288   (default)
  res512         M = 1536, the first four shapes, ternary g=64
  res512_binary  the same, binary g=64
  sweep          the 80 quantised GEMMs of one denoise step at 1024x1024 (60 launches)
  skinny         the same 80 GEMMs at M = 16 (HBM-bound; reports GB/s)

Prints one JSON line.  Inputs are seeded and synthetic: X ~ N(0,1) -> bf16, codes i.i.d.
ternary {-1:.25, 0:.5, +1:.25} (binary {-1,+1} at .5), scales U[0.005, 0.05] -> fp16.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
# Source files of each kernel variant (plus the shared headers): the committed HBM counter
# summary of a workload is used only while the sources of the kernels it runs are unchanged.
VARIANT_SOURCES = {
    "tile256x256": ["gemm_tiled.hip"], "tile256x128": ["gemm_tiled.hip"], "tile128x256": ["gemm_tiled.hip"],
    "tile64x256": ["gemm_tiled.hip"], "tile288x192": ["gemm_tile16.hip"], "tile96x192": ["gemm_tile16.hip"],
    "tile96x192k2": ["gemm_tile16.hip"], "tile64x128k2": ["gemm_tile16.hip"], "tile256x192": ["gemm_tile16.hip"],
    "tile256x256sk": ["gemm_tiled.hip"],
    "skinny": ["gemm_skinny.hip"],
    "resident": ["gemm_resident.hip"],
}
COMMON_SOURCES = ["lowbit_device.h", "lowbit_internal.h", "gemm_grouped.hip"]


def strip_comments(src: str) -> str:
    """Source text without comments, trailing blanks and empty lines (the sources hold no
    string literal with a comment marker in it)."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_sha(variants, read=None) -> str:
    """sha256 over the code (comments stripped) of the sources the variants are built from."""
    import hashlib
    files = sorted({f for v in variants for f in VARIANT_SOURCES.get(v, [])} | set(COMMON_SOURCES))
    if read is None:
        def read(rel):
            with open(os.path.join(ROOT, "binary_bit_gemm_amd", "csrc", rel)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for rel in files:
        h.update(strip_comments(read(rel)).encode())
    return h.hexdigest()


def variant_of_trace_line(line: str):
    """The kernel variant name of one LOWBIT_TRACE line ("lowbit: <family> <tile or plan> ..."),
    or None for other lines.  The 16x16-block tiles name their K split as waves=MxNxK; a stream-K
    launch of the 256 x 256 tile says "streamk" after its waves."""
    import re
    m = re.match(r"lowbit: (\w+) (\S+)(?: waves=(\d+)x(\d+)(?:x(\d+))?)?", line)
    if not m:
        return None
    family, tile, ksplit = m.group(1), m.group(2), m.group(5)
    if family in ("resident", "skinny"):
        return family
    if family == "tile16" and (ksplit == "2" or tile == "64x128"):
        return f"tile{tile}k2"  # 64 x 128 runs under that variant name with or without the split
    if family == "tiled32" and " streamk" in line:
        return f"tile{tile}sk"
    return f"tile{tile}"


def launched_variants(run_step):
    """The GEMM kernel variants one step launches, read from the library's launch log
    (LOWBIT_TRACE) with stderr sent to a temporary file around that one step; grouped calls can
    launch another tile than their problems' single calls would."""
    import tempfile
    import torch
    torch.cuda.synchronize()
    sys.stderr.flush()
    saved_fd, saved_env = os.dup(2), os.environ.get("LOWBIT_TRACE")
    with tempfile.TemporaryFile() as log:
        os.dup2(log.fileno(), 2)
        os.environ["LOWBIT_TRACE"] = "1"
        try:
            run_step()
            torch.cuda.synchronize()
        finally:
            if saved_env is None:
                os.environ.pop("LOWBIT_TRACE", None)
            else:
                os.environ["LOWBIT_TRACE"] = saved_env
            os.dup2(saved_fd, 2)
            os.close(saved_fd)
        log.seek(0)
        lines = log.read().decode(errors="replace").splitlines()
    return sorted({v for v in (variant_of_trace_line(l) for l in lines) if v is not None})


def measured_traffic(workload: str, variants):
    """HBM bytes per launch of the workload's kernels from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what it reads for a plain copy), or
    None when there is none for this workload or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sha") != kernel_source_sha(variants):
        return None
    return rec.get("bytes_per_launch")


PEAK_HBM_GBS = 8000.0
METRIC = "lowbit GEMM TFLOP/s and % of bf16 MFMA peak (M=4608, ternary g=64)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="res1024",
                    choices=["res1024", "res1024_binary", "res512", "res512_binary", "sweep", "skinny", "swiglu",
                             "swiglu16", "residual", "te4", "te4_sym"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ramp-ms", type=float, default=50.0,
                    help="untimed run of the step before the warm-up steps, so that the timed steps "
                         "find the GPU at its sustained clock (0: none)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of X in the CPU oracle sample (0 = all rows of the workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle sample until it has run this long")
    ap.add_argument("--graph", action="store_true",
                    help="launch each step as one captured HIP graph (measured slightly slower than eager launches "
                         "on these workloads, so off by default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def problems_for(workload):
    import workloads as W
    if workload == "res1024":
        return W.RES1024_TERNARY
    if workload == "res512":
        return W.RES512_TERNARY
    if workload == "res512_binary":
        return W.RES512_BINARY
    if workload == "res1024_binary":
        return W.RES1024_BINARY_G128
    if workload == "sweep":
        return W.denoise_step_sweep()
    if workload == "skinny":
        return W.denoise_step_sweep(skinny_m=16)
    if workload == "swiglu":
        # the MLP-in linear at 1024^2 (M = 4608, [gate | up] = 2 x 9216 weight rows, K = 3072) with
        # its SwiGLU fused: Y is [4608, 9216]
        return [W.Problem("m4608_mlp_in_swiglu", 4608, 18432, 3072, W.TERNARY, 64, 3, 2)]
    if workload == "residual":
        # the MLP-out linear at 1024^2 (M = 4608, 9216 -> 3072) with its gated residual update fused
        return [W.Problem("m4608_mlp_out_residual", 4608, 3072, 9216, W.TERNARY, 64, 3, 3)]
    if workload in ("te4", "te4_sym"):
        # the 4-bit text encoder's MLP at a 512-token prompt (hidden 2560, intermediate 9728): gate
        # and up fused into one 2560 -> 19456 linear, then down 9728 -> 2560; two dependent launches.
        # te4: affine groups (levels 0..15, a scale and a bias per group of 64); te4_sym: the
        # symmetric signed form
        affine = workload == "te4"
        return [W.Problem("te_mlp_gate_up", 512, 19456, 2560, W.INT4, 64, 6, 0, affine=affine),
                W.Problem("te_mlp_down", 512, 2560, 9728, W.INT4, 64, 6, 1, affine=affine)]
    if workload == "swiglu16":
        # the same linear at M = 16 (the skinny denoise-step row count)
        return [W.Problem("m16_mlp_in_swiglu", 16, 18432, 3072, W.TERNARY, 64, 3, 2)]
    raise ValueError(workload)


def swiglu_bytes(p):
    """Algorithmic bytes of a fused SwiGLU problem: Y has half the columns of the weight rows."""
    return p.bytes_moved() - p.M * (p.N // 2) * 2


def residual_bytes(p):
    """Algorithmic bytes of a fused gated-residual problem: the GEMM's, plus R read and the gate."""
    return p.bytes_moved() + p.M * p.N * 2 + p.N * 2


def make_device_inputs(probs, seed):
    """Seeded synthetic inputs drawn on the device (same distributions as workloads.py),
    codes packed with lowbit_pack (load-time, untimed)."""
    import torch
    import binary_bit_gemm_amd as lb
    gen = torch.Generator(device="cuda")
    lut = torch.tensor([-1, 0, 0, 1], dtype=torch.int8, device="cuda")
    bufs = []
    biases = {}  # affine problems: fp16 group biases
    for i, p in enumerate(probs):
        gen.manual_seed(seed * 1000003 + p.config_id * 1009 + p.tensor_id)
        x = torch.randn((p.M, p.K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        if p.affine:
            levels = torch.randint(0, 16, (p.N, p.K), generator=gen, device="cuda", dtype=torch.uint8)
            words, _ = lb.pack_u4(levels, count_invalid=False)
            del levels
            s = (torch.rand((p.N, p.K // p.g), generator=gen, device="cuda") * 0.045 + 0.005).to(torch.float16)
            biases[i] = (torch.rand((p.N, p.K // p.g), generator=gen, device="cuda") * -0.42 - 0.03).to(torch.float16)
            y = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
            bufs.append((x, words, s, y, p.g, p.bits))
            continue
        if p.bits == 2:
            codes = lut[torch.randint(0, 4, (p.N, p.K), generator=gen, device="cuda")]
        elif p.bits == 4:
            codes = torch.randint(-8, 8, (p.N, p.K), generator=gen, device="cuda", dtype=torch.int8)
        else:
            codes = (torch.randint(0, 2, (p.N, p.K), generator=gen, device="cuda", dtype=torch.int8) * 2 - 1)
        words, _ = lb.pack(codes.contiguous(), p.bits, count_invalid=False)
        del codes
        s = (torch.rand((p.N, p.K // p.g), generator=gen, device="cuda") * 0.045 + 0.005).to(torch.float16)
        y = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        bufs.append((x, words, s, y, p.g, p.bits))
    torch.cuda.synchronize()
    return bufs, biases


def cpu_baseline(probs, rows, seed, unit="TFLOP/s", min_seconds=10.0, swiglu=False):
    """The oracle as it stands (unpack, fp64 dequantise, numpy matmul) on the first `rows`
    rows of X for every distinct shape of the workload, on the host's cores, in the unit of
    the metric (TFLOP/s of 2*M*N*K, or GB/s of the algorithmic bytes of the sampled GEMMs)."""
    import numpy as np
    import oracle
    import workloads as W
    host = host_info()
    threads = host["blas_threads"]
    seen = {}
    for p in probs:
        seen.setdefault((p.N, p.K, p.bits, p.g), p)
    cases = []
    for (N, K, bits, g), p in seen.items():
        m = p.M if rows <= 0 else min(rows, p.M)
        q = W.Problem(p.name, m, N, K, bits, g, p.config_id, p.tensor_id, affine=p.affine)
        inp = W.make_inputs(q, seed)
        words, _ = oracle.pack_u4(inp.codes) if q.affine else oracle.pack(inp.codes, bits)
        cases.append((q, inp, words))
    # whole passes over the sample until at least `min_seconds` of oracle time
    flops = nbytes = passes = 0
    elapsed = 0.0
    while passes == 0 or elapsed < min_seconds:
        for q, inp, words in cases:
            t0 = time.perf_counter()
            if swiglu:
                oracle.swiglu_ref_f64(inp.x, oracle.unpack(words, q.K, q.bits), inp.scales, q.g)
            elif q.affine:
                oracle.gemm_affine_ref_f64(inp.x, oracle.unpack_u4(words, q.K), inp.scales, inp.biases, q.g)
            else:
                oracle.gemm_ref_from_words(inp.x, words, inp.scales, q.K, q.g, q.bits)
            elapsed += time.perf_counter() - t0
            flops += 2 * q.M * q.N * q.K
            nbytes += swiglu_bytes(q) if swiglu else q.bytes_moved()
        passes += 1
    value = flops / elapsed / 1e12 if unit == "TFLOP/s" else nbytes / elapsed / 1e9
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": (f"all {probs[0].M}" if rows <= 0 else f"first {rows}") +
                      f" rows of X for each of the {len(seen)} distinct (N, K) shapes, {passes} passes; "
                      f"numpy unpack + fp64 dequantise + fp64 matmul; {elapsed:.1f} s",
            "host": host}


def host_info():
    """The host the CPU baseline runs on: CPU model, logical CPUs the OS reports, CPUs this
    process may run on (affinity), and the BLAS library numpy calls with its thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            d = libs[0]
            blas = f"{d.get('internal_api')} {d.get('version')}"
            threads = d.get("num_threads")
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas": blas,
            "blas_threads": threads or affinity or os.cpu_count() or 1,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import binary_bit_gemm_amd as lb

    if a.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2}))
        return

    import workloads as W
    probs = problems_for(a.workload)
    groups = W.step_groups(probs) if a.workload in ("sweep", "skinny") else [[i] for i in range(len(probs))]
    bufs, biases = make_device_inputs(probs, a.seed)
    swiglu = a.workload in ("swiglu", "swiglu16")
    residual = a.workload == "residual"
    if residual:  # residual stream R (N(0,1)) and a per-feature gate, drawn once
        x0, w0 = bufs[0][0], bufs[0][1]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(a.seed + 77)
        res_r = torch.randn((x0.shape[0], w0.shape[0]), generator=gen, device="cuda").to(torch.bfloat16)
        res_g = torch.randn((w0.shape[0],), generator=gen, device="cuda").to(torch.bfloat16)
    if swiglu:  # the fused SwiGLU writes half the columns
        x, w, s, _, g, bits = bufs[0]
        bufs[0] = (x, w, s, torch.empty((x.shape[0], w.shape[0] // 2), dtype=torch.bfloat16, device="cuda"), g, bits)

    # one caller workspace (zero-filled once, reused by every call: each call leaves its
    # counters at zero) for the calls that split K across workgroups
    need = 0
    for grp in groups:
        if len(grp) == 1 and grp[0] in biases:
            p = probs[grp[0]]
            need = max(need, lb.affine_workspace_size(p.M, p.N, p.K, p.g))
        elif len(grp) == 1:
            p = probs[grp[0]]
            need = max(need, lb.workspace_size(p.M, p.N, p.K, p.g, p.bits))
        else:
            need = max(need, lb.batched_workspace_size([bufs[i] for i in grp]))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda") if need > 0 else None

    def launch(grp):
        if swiglu:
            x, w, s, y, g, bits = bufs[grp[0]]
            lb.gemm_swiglu(x, w, s, g, bits, out=y)
        elif residual:
            x, w, s, y, g, bits = bufs[grp[0]]
            lb.gemm_residual(x, w, s, g, bits, res_r, res_g, out=y)
        elif len(grp) == 1 and grp[0] in biases:
            x, w, s, y, g, bits = bufs[grp[0]]
            lb.gemm_affine(x, w, s, biases[grp[0]], g, out=y, workspace=ws)
        elif len(grp) == 1:
            x, w, s, y, g, bits = bufs[grp[0]]
            lb.gemm(x, w, s, g, bits, out=y, workspace=ws)
        else:
            lb.gemm_batched([bufs[i] for i in grp], workspace=ws)

    def step():
        for grp in groups:
            launch(grp)

    variants = launched_variants(step)  # one untimed step with the launch log on

    # optionally the step as one HIP graph (captured on a side stream, replayed on the current one)
    graph = None
    if a.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    run_step = graph.replay if graph is not None else step

    # Clock ramp, then the W warm-up steps, back to back: under continuous load the GPU's clock
    # rises over the first ~15 ms (per-step HIP events of res1024: 1.43 ms per step at first,
    # 1.31 ms from about the twelfth step on), so a short warm-up leaves the first timed steps
    # on a rising clock.  The step runs for about --ramp-ms first (a step count from one timed
    # step), and only the synchronisation of the timed region separates the warm-up from it.
    ramp_steps = 0
    if a.ramp_ms > 0:
        r0 = time.perf_counter()
        run_step()
        torch.cuda.synchronize()
        ramp_steps = int(a.ramp_ms / max((time.perf_counter() - r0) * 1e3, 1e-3)) + 1
    for _ in range(ramp_steps + a.warmup):
        run_step()

    # timed region: exactly `steps` steps between two synchronisations, bracketed by HIP
    # events on the stream the launches go to
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    event_ms = e0.elapsed_time(e1) / a.steps

    # per-call kernel durations with HIP events around each eager call (separate pass; the
    # breakdown only -- host launch time can show up in it for calls of a few microseconds)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
          for _ in range(a.steps)]
    for k in range(a.steps):
        for i, grp in enumerate(groups):
            ev[k][i][0].record(stream)
            launch(grp)
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(a.steps)) / a.steps
               for i in range(len(groups))]

    flops_step = sum(p.flops for p in probs)
    bytes_step = sum(swiglu_bytes(p) if swiglu else residual_bytes(p) if residual else p.bytes_moved() for p in probs)
    ms_per_step = elapsed * 1e3 / a.steps
    tflops = flops_step / (elapsed / a.steps) / 1e12
    launches = len(groups)
    # dominant kernel: every launch of the step is the same kernel family; its average launch
    # duration is the event-timed step divided by the launches per step
    launch_ms = event_ms / launches
    kern_tflops = flops_step / (event_ms * 1e-3) / 1e12
    kern_gbs = bytes_step / (event_ms * 1e-3) / 1e9
    traffic = measured_traffic(a.workload, variants)

    if a.workload in ("skinny", "swiglu16"):
        metric = ("lowbit GEMM GB/s and % of HBM peak (M=16 denoise-step sweep, ternary g=64)" if a.workload == "skinny"
                  else "lowbit fused SwiGLU GB/s and % of HBM peak (M=16 MLP-in, ternary g=64)")
        value, unit = bytes_step / (elapsed / a.steps) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(kern_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        metric = METRIC if a.workload == "res1024" else METRIC.replace("(M=4608, ternary g=64)", f"({a.workload})")
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(kern_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    roof.update({"kernel": variants, "kernel_sha": kernel_source_sha(variants),
                 "launches_per_step": launches, "avg_launch_us": round(1e3 * launch_ms, 2),
                 "algorithmic_flop_per_launch": flops_step // launches,
                 "algorithmic_bytes_per_launch": bytes_step // launches})
    out = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "gemms_per_step": len(probs), "launches_per_step": launches,
                   "workspace_bytes": need,
                   "graph": graph is not None, "clock_ramp_steps": ramp_steps,
                   "shapes": sorted({f"{p.M}x{p.N}x{p.K}" for p in probs}),
                   "bits": sorted({p.bits for p in probs}), "g": sorted({p.g for p in probs}),
                   "flop_per_step": flops_step, "bytes_per_step": bytes_step,
                   "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                   "pct_hbm_peak": round(100 * bytes_step / (elapsed / a.steps) / 1e9 / PEAK_HBM_GBS, 2),
                   "per_call_us": [round(1e3 * t, 2) for t in call_ms[:8]]},
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(probs, a.cpu_rows, a.seed, unit, a.cpu_seconds, swiglu=swiglu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
