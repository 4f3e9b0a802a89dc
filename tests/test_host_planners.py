"""Host-side planning code swept over many shapes (CPU only, no device): argument checks, the
kernel choice, the split-K planner and its workspace sizes, the grouped planner, and the early
returns of the allocation-free entry point.  The invariants checked are the ones the kernels rely
on; tests/test_host_sanitizers.py runs this file again against the library built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code."""
from __future__ import annotations

import itertools

import pytest

import binary_bit_gemm_amd as lb

OK, INVALID, UNSUPPORTED, ALIGN = 0, 1, 2, 3
COUNTER_BYTES = 4096
KNOWN = {"skinny", "resident", "tile256x128", "tile256x256", "tile128x256", "tile64x256", "tile288x192",
         "tile256x192", "tile96x192", "tile96x192k2", "tile64x128k2"}

MS = [0, 1, 2, 7, 15, 16, 17, 31, 32, 33, 64, 300, 512, 1024, 1535, 1536, 4096, 4608, 9000]
NS = [0, 16, 48, 256, 272, 1040, 3072, 9216, 18432, 27648, 36864]
KS = [0, 64, 128, 256, 320, 2560, 3072, 4352, 4608, 6144, 9216, 9728, 12288, 16384, 65536]


def test_variant_and_workspace_sweep():
    L = lb.lib()
    for M, N, K, g, bits in itertools.product(MS, NS, KS, (32, 64, 128), (1, 2, 4)):
        st = L.lowbit_check_gemm_args(256, 256, 256, 256, M, N, K, g, bits)
        if bits == 4 and g == 32:
            assert st == UNSUPPORTED
            continue
        if K % g:
            assert st == INVALID, (M, N, K, g, bits)
            continue
        assert st == OK, (M, N, K, g, bits, st)
        if M * N * K == 0:
            continue
        v = lb.variant(M, N, K, g, bits)
        assert v in KNOWN, (M, N, K, g, bits, v)
        if bits == 4:
            assert v in ("tile288x192", "tile256x192", "tile96x192", "tile96x192k2", "tile64x128k2"), v
        ws = lb.workspace_size(M, N, K, g, bits)
        if ws:
            # only skinny ternary shapes split K, and every automatic plan fits the static scratch
            assert bits == 2 and M <= 16 and g in (64, 128) and K % 256 == 0, (M, N, K, g, bits)
            assert COUNTER_BYTES < ws <= lb.NOALLOC_SCRATCH_BYTES
            assert (ws - COUNTER_BYTES) % 1024 == 0


def test_limits_and_overflow_edges():
    L = lb.lib()
    big = (1 << 31) - 1
    cases = [
        ((16, big - 15, 64, 64, 2), UNSUPPORTED),       # packed weights past 4 GiB
        ((16, big, 64, 64, 2), INVALID),                # N % 16
        ((big, 16, 64, 64, 2), OK),
        ((1 << 31, 16, 64, 64, 2), INVALID),
        ((16, 16, (1 << 22) + 64, 64, 2), UNSUPPORTED),  # K past 2^22
        ((16, 16, 1 << 22, 64, 2), OK),
        ((1 << 20, 1 << 18, 64, 64, 2), UNSUPPORTED),    # M * N past 2^37
        ((-1, 16, 64, 64, 2), INVALID),
        ((16, -16, 64, 64, 2), INVALID),
        ((16, 16, -64, 64, 2), INVALID),
        ((16, 16, 64, 48, 2), UNSUPPORTED),
        ((16, 16, 64, 64, 3), UNSUPPORTED),
        ((16, 24, 64, 64, 2), INVALID),
    ]
    for (M, N, K, g, bits), want in cases:
        assert L.lowbit_check_gemm_args(256, 256, 256, 256, M, N, K, g, bits) == want, (M, N, K, g, bits)
        # the size queries stay defined (0 for what no kernel takes)
        assert lb.workspace_size(M, N, K, g, bits) >= 0
        if want != OK:
            assert L.lowbit_gemm_noalloc(256, 256, 256, 256, M, N, K, g, bits, None) == want


@pytest.mark.parametrize("plan", ["1,2", "4,3", "16,16", "6,48", "9,4", "1,16", "2,1000"])
def test_forced_split_plans(plan, monkeypatch):
    """Forced split plans keep their workspace inside the fixed counter region's tile limit and
    the documented size (counters + tiles x splits x column blocks x 1 KiB)."""
    monkeypatch.setenv("LOWBIT_RESIDENT_PLAN", plan)
    cb, splits = (int(v) for v in plan.split(","))
    for N, K in [(256, 6144), (3072, 12288), (16384, 16384), (18432, 9216), (65536, 4096)]:
        ws = lb.workspace_size(16, N, K, 64, 2)
        if ws == 0:
            continue
        tiles = -(-(N // 16) // cb)
        assert tiles <= 1024, (plan, N, K)
        s = min(splits, K // 256)
        assert ws == COUNTER_BYTES + tiles * s * cb * 1024, (plan, N, K, ws)


def test_grouped_planner_sweep():
    L = lb.lib()
    A = 256
    pairs = [(4096, 512), (16, 16), (1, 16), (16, 4608), (300, 7)]
    for (m1, m2), (N, K), g in itertools.product(pairs, [(9216, 3072), (3072, 9216), (3072, 12288), (18432, 3072),
                                                         (256, 6144)], (64, 128)):
        arr = (lb.Problem * 2)()
        arr[0] = lb.Problem(A, A, A, A, m1, N, K, g, 2)
        arr[1] = lb.Problem(A, A, A, A, m2, N, K, g, 2)
        ws = L.lowbit_batched_workspace_size(arr, 2)
        assert ws == 0 or COUNTER_BYTES < ws <= 2 * lb.NOALLOC_SCRATCH_BYTES
        if min(m1, m2) > 16:  # only skinny problems split K
            assert ws == 0
    # the largest batch: LOWBIT_MAX_BATCH problems of mixed classes
    arr = (lb.Problem * lb.MAX_BATCH)()
    for i in range(lb.MAX_BATCH):
        arr[i] = lb.Problem(A, A, A, A, (i % 5) * 7 + 1, 16 * (i + 1), 256 * (1 + i % 3), (64, 128)[i % 2], (1, 2)[i % 2])
    assert L.lowbit_batched_workspace_size(arr, lb.MAX_BATCH) >= 0
    assert L.lowbit_batched_workspace_size(arr, lb.MAX_BATCH + 1) == 0
