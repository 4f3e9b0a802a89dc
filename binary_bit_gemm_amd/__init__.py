"""binary_bit_gemm_amd -- packed ternary / binary weight GEMM for AMD MI355X (gfx950).

Thin ctypes binding over liblowbit.so (include/lowbit.h).  Every step of the computation
runs in the library's HIP kernels; this module only checks tensor types, takes device
pointers and the current HIP stream, and raises on a non-zero status.  PyTorch is used for
device memory and streams only.

    import torch, binary_bit_gemm_amd as lb
    words, bad = lb.pack(codes_int8_cuda, bits=2)          # [N, K] -> [N, K/16] (int32 view)
    y = lb.gemm(x_bf16_cuda, words, scales_fp16_cuda, g=64, bits=2)
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

from ._lib import LowbitError, lib, library_path  # noqa: F401

TERNARY = 2
BINARY = 1
MAX_BATCH = 64


def _torch():
    import torch
    return torch


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        msg = L.lowbit_status_string(status).decode()
        hip = L.lowbit_last_hip_error()
        raise LowbitError(status, f"{what}: {msg}" + (f" (hipError {hip})" if status == 4 else ""))


def _require(t, dtype, name: str, ndim: int = 2):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def words_per_row(K: int, bits: int) -> int:
    return K * bits // 32


def pack(codes, bits: int, count_invalid: bool = True) -> Tuple["object", Optional[int]]:
    """int8 codes [N, K] on the GPU -> (packed words [N, K*bits/32] as int32, invalid count).

    The invalid count (codes outside {-1,0,1} / {-1,1}) is read back only when
    count_invalid is true (that synchronises the stream)."""
    torch = _torch()
    _require(codes, torch.int8, "codes")
    N, K = codes.shape
    words = torch.empty((N, words_per_row(K, bits)), dtype=torch.int32, device=codes.device)
    bad = torch.zeros(1, dtype=torch.int32, device=codes.device) if count_invalid else None
    st = lib().lowbit_pack(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(words.data_ptr()), N, K, bits,
                           ctypes.c_void_p(bad.data_ptr() if bad is not None else 0),
                           ctypes.c_void_p(_stream_ptr(codes.device)))
    _check(st, "lowbit_pack")
    return words, (int(bad.item()) if bad is not None else None)


def pack_u4(levels, count_invalid: bool = True):
    """Unsigned 4-bit levels (uint8 [N, K], 0 .. 15) on the GPU -> (packed words [N, K/8] as
    int32, invalid count) for lowbit_gemm_affine (lowbit_pack_u4)."""
    torch = _torch()
    _require(levels, torch.uint8, "levels")
    N, K = levels.shape
    words = torch.empty((N, K // 8), dtype=torch.int32, device=levels.device)
    bad = torch.zeros(1, dtype=torch.int32, device=levels.device) if count_invalid else None
    st = lib().lowbit_pack_u4(ctypes.c_void_p(levels.data_ptr()), ctypes.c_void_p(words.data_ptr()), N, K,
                              ctypes.c_void_p(bad.data_ptr() if bad is not None else 0),
                              ctypes.c_void_p(_stream_ptr(levels.device)))
    _check(st, "lowbit_pack_u4")
    return words, (int(bad.item()) if bad is not None else None)


def affine_workspace_size(M: int, N: int, K: int, g: int = 64) -> int:
    """Bytes of workspace lowbit_gemm_affine_ex can use for this shape (0: it takes no split)."""
    return int(lib().lowbit_affine_workspace_size(M, N, K, g))


def gemm_affine(x, words, scales, biases, g: int, out=None, workspace=None):
    """Y = X . W^T with affine 4-bit groups W = S * q + B (lowbit_gemm_affine): `words` from
    pack_u4, `scales` and `biases` fp16 [N, K/g].  `workspace`: an optional zero-filled device
    tensor of at least affine_workspace_size(M, N, K, g) bytes (lowbit_gemm_affine_ex), with which
    shapes whose tile grid leaves compute units idle split K across workgroups."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    _require(words, torch.int32, "words")
    _require(scales, torch.float16, "scales")
    _require(biases, torch.float16, "biases")
    M, K = x.shape
    N = words.shape[0]
    if words.shape[1] != K // 8 or K % 8:
        raise ValueError(f"words must be [N, K/8] = [{N}, {K // 8}], got {tuple(words.shape)}")
    if K % g or tuple(scales.shape) != (N, K // g) or tuple(biases.shape) != (N, K // g):
        raise ValueError(f"scales and biases must be [N, K/g] = [{N}, {K // g if g else 0}]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, torch.bfloat16, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    args = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
            ctypes.c_void_p(biases.data_ptr()), ctypes.c_void_p(out.data_ptr()), M, N, K, g)
    if workspace is None:
        st = lib().lowbit_gemm_affine(*args, ctypes.c_void_p(_stream_ptr(x.device)))
        _check(st, "lowbit_gemm_affine")
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        nbytes = workspace.numel() * workspace.element_size()
        st = lib().lowbit_gemm_affine_ex(*args, ctypes.c_void_p(workspace.data_ptr()), nbytes,
                                         ctypes.c_void_p(_stream_ptr(x.device)))
        _check(st, "lowbit_gemm_affine_ex")
    return out


def unpack(words, K: int, bits: int):
    """Packed words [N, K*bits/32] -> int8 codes [N, K]."""
    torch = _torch()
    _require(words, torch.int32, "words")
    N = words.shape[0]
    if words.shape[1] != words_per_row(K, bits):
        raise ValueError("words do not hold K codes per row")
    codes = torch.empty((N, K), dtype=torch.int8, device=words.device)
    st = lib().lowbit_unpack(ctypes.c_void_p(words.data_ptr()), ctypes.c_void_p(codes.data_ptr()), N, K, bits,
                             ctypes.c_void_p(_stream_ptr(words.device)))
    _check(st, "lowbit_unpack")
    return codes


LAYOUT_GEMLITE_U8T = 1  # uint8 [K/4, N]: GemLite's int2 weights, packed over K with a transpose
LAYOUT_MLX_U32 = 2      # uint32 [N, K/16]: MLX's packed rows


def _import(src, layout: int, N: int, K: int, zero: int, count_invalid: bool):
    torch = _torch()
    words = torch.empty((N, words_per_row(K, 2)), dtype=torch.int32, device=src.device)
    bad = torch.zeros(1, dtype=torch.int32, device=src.device) if count_invalid else None
    st = lib().lowbit_import_ternary(ctypes.c_void_p(src.data_ptr()), layout, zero, ctypes.c_void_p(words.data_ptr()),
                                     N, K, ctypes.c_void_p(bad.data_ptr() if bad is not None else 0),
                                     ctypes.c_void_p(_stream_ptr(src.device)))
    _check(st, "lowbit_import_ternary")
    return words, (int(bad.item()) if bad is not None else None)


def import_gemlite(src, N: int, K: int, zero: int = 1, count_invalid: bool = True):
    """GemLite int2 weights, uint8 [K/4, N] (transposed), levels q with code q - zero ->
    (packed words [N, K/16] as int32, invalid count).  N and K are the caller's: the
    orientation is never guessed from the buffer's shape, which is checked against them."""
    torch = _torch()
    _require(src, torch.uint8, "src")
    if tuple(src.shape) != (K // 4, N) or K % 4:
        raise ValueError(f"GemLite src must be uint8 [K/4, N] = ({K // 4}, {N}), got {tuple(src.shape)}")
    return _import(src, LAYOUT_GEMLITE_U8T, N, K, zero, count_invalid)


def import_mlx(src, N: int, K: int, zero: int = 1, count_invalid: bool = True):
    """MLX 2-bit rows, uint32 (or int32) [N, K/16], levels q with code q - zero -> (packed words
    [N, K/16] as int32, invalid count)."""
    torch = _torch()
    _require(src, torch.uint32 if src.dtype == torch.uint32 else torch.int32, "src")
    if tuple(src.shape) != (N, K // 16) or K % 16:
        raise ValueError(f"MLX src must be [N, K/16] = ({N}, {K // 16}), got {tuple(src.shape)}")
    return _import(src, LAYOUT_MLX_U32, N, K, zero, count_invalid)


def import_gemlite_binary(src, N: int, K: int):
    """GemLite 1-bit weights, uint8 [K/8, N] (transposed, bit i of byte (j, n) = code 8j + i,
    1 -> +1) -> packed binary words [N, K/32] as int32."""
    torch = _torch()
    _require(src, torch.uint8, "src")
    if tuple(src.shape) != (K // 8, N) or K % 8:
        raise ValueError(f"GemLite 1-bit src must be uint8 [K/8, N] = ({K // 8}, {N}), got {tuple(src.shape)}")
    words = torch.empty((N, words_per_row(K, 1)), dtype=torch.int32, device=src.device)
    st = lib().lowbit_import_binary_gemlite(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(words.data_ptr()), N, K,
                                            ctypes.c_void_p(_stream_ptr(src.device)))
    _check(st, "lowbit_import_binary_gemlite")
    return words


def workspace_size(M: int, N: int, K: int, g: int = 64, bits: int = 2) -> int:
    """Bytes of workspace lowbit_gemm_ex can use for this shape (0: none needed)."""
    return int(lib().lowbit_workspace_size(M, N, K, g, bits))


def gemm(x, words, scales, g: int, bits: int, out=None, workspace=None):
    """Y[M, N] = X[M, K] . dequant(W)[N, K]^T in bf16 (see include/lowbit.h).

    `workspace`: an optional zero-filled device tensor (any dtype) of at least
    workspace_size(M, N, K, g, bits) bytes; it lets skinny problems split K across
    workgroups (lowbit_gemm_ex).  Reuse it between calls; do not share it between calls
    that run concurrently."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    _require(words, torch.int32, "words")
    _require(scales, torch.float16, "scales")
    M, K = x.shape
    N = words.shape[0]
    if words.shape[1] != words_per_row(K, bits):
        raise ValueError(f"words must be [N, K*bits/32] = [{N}, {words_per_row(K, bits)}], got {tuple(words.shape)}")
    if K % g or tuple(scales.shape) != (N, K // g):
        raise ValueError(f"scales must be [N, K/g] = [{N}, {K // g if g else 0}], got {tuple(scales.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, torch.bfloat16, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    if workspace is None:
        st = lib().lowbit_gemm(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()),
                               ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                               M, N, K, g, bits, ctypes.c_void_p(_stream_ptr(x.device)))
        _check(st, "lowbit_gemm")
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        nbytes = workspace.numel() * workspace.element_size()
        st = lib().lowbit_gemm_ex(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()),
                                  ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  M, N, K, g, bits, ctypes.c_void_p(workspace.data_ptr()), nbytes,
                                  ctypes.c_void_p(_stream_ptr(x.device)))
        _check(st, "lowbit_gemm_ex")
    return out


NOALLOC_SCRATCH_BYTES = 4096 + 512 * 16 * 1024  # LOWBIT_NOALLOC_SCRATCH_BYTES of include/lowbit.h


def gemm_noalloc(x, words, scales, g: int, bits: int, out):
    """lowbit_gemm_noalloc: lowbit_gemm_ex on the library's static per-GPU scratch, for callers
    that cannot allocate (`out` is required: this call allocates nothing).  Calls on one GPU
    share the scratch and must not overlap."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    _require(words, torch.int32, "words")
    _require(scales, torch.float16, "scales")
    _require(out, torch.bfloat16, "out")
    M, K = x.shape
    N = words.shape[0]
    if words.shape[1] != words_per_row(K, bits):
        raise ValueError(f"words must be [N, K*bits/32] = [{N}, {words_per_row(K, bits)}], got {tuple(words.shape)}")
    if K % g or tuple(scales.shape) != (N, K // g):
        raise ValueError(f"scales must be [N, K/g] = [{N}, {K // g if g else 0}], got {tuple(scales.shape)}")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    st = lib().lowbit_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()),
                                   ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                   M, N, K, g, bits, ctypes.c_void_p(_stream_ptr(x.device)))
    _check(st, "lowbit_gemm_noalloc")
    return out


class Problem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("W", ctypes.c_void_p), ("S", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("g", ctypes.c_int32), ("bits", ctypes.c_int32)]


def gemm_swiglu(x, words, scales, g: int, bits: int, out=None):
    """Y[M, N] = silu(X . dequant(Wg)^T) * (X . dequant(Wu)^T) in bf16, with `words` / `scales`
    holding 2N rows: gate rows [0, N), then up rows [N, 2N) (lowbit_gemm_swiglu)."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    _require(words, torch.int32, "words")
    _require(scales, torch.float16, "scales")
    M, K = x.shape
    N2 = words.shape[0]
    if N2 % 2:
        raise ValueError(f"words must hold 2N rows (gate then up), got {N2}")
    N = N2 // 2
    if words.shape[1] != words_per_row(K, bits):
        raise ValueError(f"words must be [2N, K*bits/32] = [{N2}, {words_per_row(K, bits)}], got {tuple(words.shape)}")
    if K % g or tuple(scales.shape) != (N2, K // g):
        raise ValueError(f"scales must be [2N, K/g] = [{N2}, {K // g if g else 0}], got {tuple(scales.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, torch.bfloat16, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    st = lib().lowbit_gemm_swiglu(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()),
                                  ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  M, N, K, g, bits, ctypes.c_void_p(_stream_ptr(x.device)))
    _check(st, "lowbit_gemm_swiglu")
    return out


def gemm_residual(x, words, scales, g: int, bits: int, residual, gate, out=None):
    """Y[M, N] = residual + gate[n] * (X . dequant(W)^T) in bf16 (lowbit_gemm_residual).
    `out` may be `residual` itself (in-place update of the residual stream)."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    _require(words, torch.int32, "words")
    _require(scales, torch.float16, "scales")
    _require(residual, torch.bfloat16, "residual")
    _require(gate, torch.bfloat16, "gate", ndim=1)
    M, K = x.shape
    N = words.shape[0]
    if words.shape[1] != words_per_row(K, bits):
        raise ValueError(f"words must be [N, K*bits/32] = [{N}, {words_per_row(K, bits)}], got {tuple(words.shape)}")
    if K % g or tuple(scales.shape) != (N, K // g):
        raise ValueError(f"scales must be [N, K/g] = [{N}, {K // g if g else 0}], got {tuple(scales.shape)}")
    if tuple(residual.shape) != (M, N) or tuple(gate.shape) != (N,):
        raise ValueError("residual must be [M, N] and gate [N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, torch.bfloat16, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    st = lib().lowbit_gemm_residual(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(words.data_ptr()),
                                    ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(residual.data_ptr()),
                                    ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                    M, N, K, g, bits, ctypes.c_void_p(_stream_ptr(x.device)))
    _check(st, "lowbit_gemm_residual")
    return out


def _problem_array(problems):
    torch = _torch()
    if len(problems) > MAX_BATCH:
        raise ValueError(f"at most {MAX_BATCH} problems per call")
    arr = (Problem * max(1, len(problems)))()
    dev = None
    for i, (x, w, s, y, g, bits) in enumerate(problems):
        _require(x, torch.bfloat16, "x")
        _require(w, torch.int32, "words")
        _require(s, torch.float16, "scales")
        _require(y, torch.bfloat16, "out")
        M, K = x.shape
        N = w.shape[0]
        if w.shape[1] != words_per_row(K, bits) or tuple(s.shape) != (N, K // g) or tuple(y.shape) != (M, N):
            raise ValueError(f"problem {i}: inconsistent shapes")
        dev = x.device
        arr[i] = Problem(x.data_ptr(), w.data_ptr(), s.data_ptr(), y.data_ptr(), M, N, K, g, bits)
    return arr, dev


def batched_workspace_size(problems: Sequence[Tuple["object", "object", "object", "object", int, int]]) -> int:
    """Bytes of workspace gemm_batched(..., workspace=...) can use (0: none needed)."""
    arr, _ = _problem_array(problems)
    return int(lib().lowbit_batched_workspace_size(arr, len(problems))) if problems else 0


def gemm_batched(problems: Sequence[Tuple["object", "object", "object", "object", int, int]],
                 workspace=None) -> None:
    """Run independent GEMMs [(x, words, scales, out, g, bits), ...] as grouped launches.
    Outputs are written in place; all tensors on the same device.  `workspace`: as for gemm()
    (size from batched_workspace_size)."""
    arr, dev = _problem_array(problems)
    if not problems:
        return
    stream = ctypes.c_void_p(_stream_ptr(dev))
    if workspace is None:
        st = lib().lowbit_gemm_batched(arr, len(problems), stream)
        _check(st, "lowbit_gemm_batched")
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        st = lib().lowbit_gemm_batched_ex(arr, len(problems), ctypes.c_void_p(workspace.data_ptr()),
                                          workspace.numel() * workspace.element_size(), stream)
        _check(st, "lowbit_gemm_batched_ex")


def check_gemm_args(x_ptr: int, w_ptr: int, s_ptr: int, y_ptr: int, M: int, N: int, K: int, g: int,
                    bits: int) -> int:
    """Host-only validation (no HIP call); returns the status code lowbit_gemm would return."""
    return lib().lowbit_check_gemm_args(ctypes.c_void_p(x_ptr), ctypes.c_void_p(w_ptr), ctypes.c_void_p(s_ptr),
                                        ctypes.c_void_p(y_ptr), M, N, K, g, bits)


def variant(M: int, N: int, K: int, g: int = 64, bits: int = 2) -> str:
    """Name of the kernel variant lowbit_gemm picks for this shape."""
    return lib().lowbit_gemm_variant(M, N, K, g, bits).decode()


def status_string(status: int) -> str:
    return lib().lowbit_status_string(status).decode()


def version() -> int:
    return lib().lowbit_version()
