"""Plain numpy/fp64 reference for the packed low-bit weight GEMM (test infrastructure only).

What is computed (model-card and guide passages cited per function):

    Y[m, n] = sum_k  X[m, k] * c[n, k] * S[n, k // g]

with X given as bf16 bit patterns, c the integer weight codes (ternary {-1, 0, +1} or
binary {-1, +1}), S the fp16 group scales, all evaluated in fp64.  Every product
bf16 * fp16 * {-1, 0, 1} has at most 8 + 11 significant bits and is exact in fp64, so
this is the exact result up to the summation order of the fp64 matmul.

Readings taken where the pages are silent (each also recorded with the format
definition in include/lowbit.h):

R1  Ternary encoding: 2-bit field 00 -> 0, 01 -> +1, 10 -> -1.  The field 11 never comes
    out of the packer; the unpacker maps it to 0 via c = (f & 1) - ((f >> 1) & 1).
R2  Word order: 16 ternary (32 binary) codes per uint32, consecutive along K, least
    significant field first: code k lives in word k // 16 at bits 2*(k % 16) .. +1
    (binary: word k // 32, bit k % 32, bit 1 -> +1, bit 0 -> -1).
R3  Layout: packed words [N, K*bits/32] and scales [N, K/g], both row-major by output
    feature n.
R4  Scale form: symmetric w = s * c for ternary too (the binary model card gives
    w = scale_g * b; no zero point is mentioned anywhere).
R5  Invalid codes handed to the packer (ternary outside {-1,0,1}, binary outside
    {-1,1}) are packed as 0 bits and counted.
R6  SwiGLU of the MLP-in linear (the MMDiT's 2 x 9216-output linear, mlx guide section
    "组件架构"): its 2N output features are [gate | up], gate first, and the activation
    is silu(gate) * up with silu(a) = a / (1 + exp(-a)).  Which half gates is not stated
    on the pages.
R7  Gated residual of a block's output linear (the mlx guide's modulated MMDiT blocks,
    section "组件架构"): Y = R + gate[n] * (X . W^T)[m, n] with a per-feature gate; the exact
    form is a reading.
R8  Importers of other runtimes' ternary packs: both hold unsigned 2-bit levels q, least
    significant field first, with code c = q - zero (zero = 1 for the symmetric form; the
    pages do not give the level coding).  GemLite: uint8 [K/4, N], byte (j, n) holding codes
    k = 4j .. 4j+3 of row n (Bonsai-Image-Demo pull request 20, "CPU bring-up": packed over
    K with a transpose, (in_features / 4, out_features)).  MLX: uint32 [N, K/16], word (n, j)
    holding codes k = 16j .. 16j+15 ("backend/ -- FastAPI Mac backend", "Checkpoint layout").
R9  4-bit codes (the 4-bit text encoder of the binary model card's "Model Overview" table):
    integers c in [-8, 7] as two's complement nibbles, 8 per uint32 along K, least significant
    first (code k at bits 4*(k % 8) of word k // 8), with the symmetric form w = s * c of R4.
    The card names only "4-bit HQQ"; its zero points are not on the pages.
R10 Affine 4-bit groups of the text encoder: the mlx guide (section "组件架构") loads the
    4-bit Qwen3 text encoder quantised with bits = 4, group_size = 64, and the CPU bring-up
    (Bonsai-Image-Demo pull request 20) dequantises the HQQ text encoder.  Both runtimes' 4-bit
    groups are affine; the plainest common form is w = s * q + b with unsigned levels
    q in [0, 15] and one fp16 scale s and one fp16 bias b per group of g consecutive weights
    along K (an HQQ zero point z is b = -z * s).  Levels are packed 8 per uint32, least
    significant nibble first (level k at bits 4*(k % 8) of word k // 8), like R9.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

TERNARY = 2
BINARY = 1
INT4 = 4

REL_FROB_TOL = 5e-3
ELEM_TOL = 1e-2


# ----------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64.  A bf16 number is the upper half of an IEEE binary32,
    so widening is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_rne(y: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 (8 significant bits, 8 exponent bits), ties to even.

    Written from the definition: split |y| = f * 2**e with f in [0.5, 1), keep 8
    significant bits by rounding |y| / 2**(e-8) to the nearest integer (numpy's rint
    rounds halves to even), with the quantum floored at bf16's subnormal spacing 2**-133;
    overflow goes to infinity.  The rounded value is representable in binary32, whose
    upper 16 bits are the bf16 pattern."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.uint16)
    a = np.abs(y)
    nz = a > 0
    f, e = np.frexp(a[nz])
    quantum_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(a[nz], -quantum_exp))
    val = np.ldexp(q, quantum_exp)
    with np.errstate(over="ignore"):
        v32 = val.astype(np.float32)
    bits = (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[val >= 2.0 ** 128] = 0x7F80
    out[nz] = bits
    out |= np.where(np.signbit(y), np.uint16(0x8000), np.uint16(0))
    return out


# ----------------------------------------------------------------------------------------
# Packing (readings R1, R2, R5)
# ----------------------------------------------------------------------------------------

def pack(codes: np.ndarray, bits: int) -> Tuple[np.ndarray, int]:
    """int8 codes [N, K] -> (uint32 words [N, K*bits/32], number of invalid codes).

    Ternary: field(c) = 01 for +1, 10 for -1, 00 for 0, placed at bits 2*(k % 16) of word
    k // 16.  Binary: bit 1 for +1, bit 0 for -1, at bit k % 32 of word k // 32.  4-bit: the
    nibble c mod 16 (two's complement) at bits 4*(k % 8) of word k // 8 (reading R9)."""
    c = np.asarray(codes, dtype=np.int8)
    if c.ndim != 2:
        raise ValueError("codes must be 2-D [N, K]")
    N, K = c.shape
    per_word = 32 // bits
    if bits not in (TERNARY, BINARY, INT4) or K % per_word:
        raise ValueError("bits must be 1, 2 or 4 and K a multiple of 32/bits")
    field = np.zeros((N, K), dtype=np.uint32)
    if bits == INT4:
        ok = (c >= -8) & (c <= 7)
        field[ok] = (c[ok].astype(np.int64) % 16).astype(np.uint32)
        bad = int(np.count_nonzero(~ok))
    elif bits == TERNARY:
        field[c == 1] = 1
        field[c == -1] = 2
        bad = int(np.count_nonzero((c != 0) & (c != 1) & (c != -1)))
    else:
        field[c == 1] = 1
        bad = int(np.count_nonzero((c != 1) & (c != -1)))
    field = field.reshape(N, K // per_word, per_word)
    words = np.zeros((N, K // per_word), dtype=np.uint32)
    for i in range(per_word):
        words |= field[:, :, i] << np.uint32(bits * i)
    return words, bad


def unpack(words: np.ndarray, K: int, bits: int) -> np.ndarray:
    """uint32 words [N, K*bits/32] -> int8 codes [N, K].

    Ternary: c = (f & 1) - ((f >> 1) & 1) for each 2-bit field f (so 11 decodes to 0).
    Binary: c = 2 * bit - 1.  4-bit: c = f - 16 for nibbles f >= 8, else f."""
    w = np.asarray(words, dtype=np.uint32)
    per_word = 32 // bits
    N = w.shape[0]
    if w.shape[1] * per_word != K:
        raise ValueError("words do not hold K codes per row")
    out = np.zeros((N, w.shape[1], per_word), dtype=np.int8)
    for i in range(per_word):
        f = (w >> np.uint32(bits * i)) & np.uint32((1 << bits) - 1)
        if bits == INT4:
            out[:, :, i] = np.where(f >= 8, f.astype(np.int64) - 16, f.astype(np.int64)).astype(np.int8)
        elif bits == TERNARY:
            out[:, :, i] = (f & 1).astype(np.int8) - ((f >> 1) & 1).astype(np.int8)
        else:
            out[:, :, i] = 2 * f.astype(np.int8) - 1
    return out.reshape(N, K)


def _level_codes(q: np.ndarray, zero: int) -> Tuple[np.ndarray, int]:
    """Unsigned levels -> ternary codes c = q - zero; codes outside {-1, 0, 1} become 0 and
    are counted (reading R8)."""
    c = q.astype(np.int64) - zero
    bad = np.abs(c) > 1
    c[bad] = 0
    return c.astype(np.int8), int(np.count_nonzero(bad))


def gemlite_u8t_decode(src: np.ndarray, N: int, K: int, zero: int = 1) -> Tuple[np.ndarray, int]:
    """GemLite transposed uint8 [K/4, N] -> (int8 codes [N, K], invalid count): code k of
    row n is the 2-bit level at bits 2*(k % 4) of byte (k // 4, n), minus `zero`."""
    b = np.asarray(src, dtype=np.uint8)
    if b.shape != (K // 4, N) or K % 4:
        raise ValueError("GemLite src must be [K/4, N]")
    q = np.zeros((N, K), dtype=np.uint8)
    for k in range(K):
        q[:, k] = (b[k // 4, :] >> (2 * (k % 4))) & 3
    return _level_codes(q, zero)


def mlx_u32_decode(src: np.ndarray, N: int, K: int, zero: int = 1) -> Tuple[np.ndarray, int]:
    """MLX uint32 rows [N, K/16] -> (int8 codes [N, K], invalid count): code k of row n is the
    2-bit level at bits 2*(k % 16) of word (n, k // 16), minus `zero`."""
    w = np.asarray(src, dtype=np.uint32)
    if w.shape != (N, K // 16) or K % 16:
        raise ValueError("MLX src must be [N, K/16]")
    q = np.zeros((N, K), dtype=np.uint32)
    for k in range(K):
        q[:, k] = (w[:, k // 16] >> np.uint32(2 * (k % 16))) & np.uint32(3)
    return _level_codes(q, zero)


def gemlite_binary_decode(src: np.ndarray, N: int, K: int) -> np.ndarray:
    """GemLite 1-bit transposed uint8 [K/8, N] -> binary codes [N, K]: code k of row n is
    2 * (bit k % 8 of byte (k // 8, n)) - 1 (reading R8 with 8 codes per byte)."""
    b = np.asarray(src, dtype=np.uint8)
    if b.shape != (K // 8, N) or K % 8:
        raise ValueError("GemLite 1-bit src must be [K/8, N]")
    out = np.zeros((N, K), dtype=np.int8)
    for k in range(K):
        out[:, k] = 2 * ((b[k // 8, :] >> (k % 8)) & 1).astype(np.int8) - 1
    return out


def gemlite_binary_encode(codes: np.ndarray) -> np.ndarray:
    """Binary codes [N, K] (+1 / -1) -> GemLite 1-bit transposed uint8 [K/8, N]."""
    c = np.asarray(codes, dtype=np.int8)
    N, K = c.shape
    if K % 8 or np.any((c != 1) & (c != -1)):
        raise ValueError("binary codes and K a multiple of 8")
    out = np.zeros((K // 8, N), dtype=np.uint8)
    for k in range(K):
        out[k // 8, :] |= ((c[:, k] == 1).astype(np.uint8) << (k % 8)).astype(np.uint8)
    return out


def gemlite_u8t_encode(codes: np.ndarray, zero: int = 1) -> np.ndarray:
    """int8 codes [N, K] -> GemLite transposed uint8 [K/4, N] with levels q = c + zero (0..3)."""
    c = np.asarray(codes, dtype=np.int64)
    N, K = c.shape
    q = c + zero
    if K % 4 or q.min(initial=0) < 0 or q.max(initial=0) > 3:
        raise ValueError("levels must lie in 0..3 and K be a multiple of 4")
    out = np.zeros((K // 4, N), dtype=np.uint8)
    for k in range(K):
        out[k // 4, :] |= (q[:, k] << (2 * (k % 4))).astype(np.uint8)
    return out


def mlx_u32_encode(codes: np.ndarray, zero: int = 1) -> np.ndarray:
    """int8 codes [N, K] -> MLX uint32 rows [N, K/16] with levels q = c + zero (0..3)."""
    c = np.asarray(codes, dtype=np.int64)
    N, K = c.shape
    q = c + zero
    if K % 16 or q.min(initial=0) < 0 or q.max(initial=0) > 3:
        raise ValueError("levels must lie in 0..3 and K be a multiple of 16")
    out = np.zeros((N, K // 16), dtype=np.uint32)
    for k in range(K):
        out[:, k // 16] |= (q[:, k] << (2 * (k % 16))).astype(np.uint32)
    return out


# ----------------------------------------------------------------------------------------
# Dequantise and matmul
# ----------------------------------------------------------------------------------------

def dequant_f64(codes: np.ndarray, scales: np.ndarray, g: int) -> np.ndarray:
    """W[n, k] = c[n, k] * S[n, k // g] in fp64 (exact).

    The model card's binary form w_i = scale_g * b_i with one fp16 scale per group of g
    consecutive weights along the input dimension; ternary takes the same symmetric
    form (reading R4)."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float64)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    N, K = c.shape
    if K % g or s.shape != (N, K // g):
        raise ValueError("scales must be [N, K // g]")
    s_per_k = np.repeat(s, g, axis=1)  # S[n, k // g] for every k
    return c * s_per_k


def gemm_ref_f64(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, g: int) -> np.ndarray:
    """Y = X @ dequant(W).T in fp64: dequantise to dense, then an ordinary matmul (the
    shape of the CPU bring-up path in the Bonsai-Image-Demo report)."""
    xd = bf16_bits_to_f64(x_bits)
    wd = dequant_f64(codes, scales, g)
    if xd.shape[1] != wd.shape[1]:
        raise ValueError("X and W disagree on K")
    return xd @ wd.T


def gemm_ref_from_words(x_bits: np.ndarray, words: np.ndarray, scales: np.ndarray,
                        K: int, g: int, bits: int) -> np.ndarray:
    """The same reference starting from packed words (unpack, dequantise, matmul)."""
    return gemm_ref_f64(x_bits, unpack(words, K, bits), scales, g)


def gemm_fsum_element(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, g: int,
                      m: int, n: int) -> float:
    """One output element as the correctly rounded sum (math.fsum) of its exact products."""
    x = bf16_bits_to_f64(np.asarray(x_bits)[m])
    c = np.asarray(codes)[n]
    s = np.asarray(scales, dtype=np.float16)[n].astype(np.float64)
    return math.fsum(float(x[k]) * int(c[k]) * float(s[k // g]) for k in range(c.shape[0]))


def silu_f64(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a)) in fp64, evaluated as a * exp(a) / (1 + exp(a))
    for negative a so that no exp overflows (reading R6)."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    e = np.exp(a[~pos])
    out[~pos] = a[~pos] * e / (1.0 + e)
    return out


def swiglu_ref_f64(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, g: int) -> np.ndarray:
    """Y[M, N] = silu(X @ Wg.T) * (X @ Wu.T) in fp64, where codes / scales hold 2N rows:
    gate rows [0, N), then up rows [N, 2N) (reading R6).  Both factors are the exact
    reference GEMM of the same rows."""
    c = np.asarray(codes)
    if c.shape[0] % 2:
        raise ValueError("SwiGLU weights hold 2N rows (gate, then up)")
    n = c.shape[0] // 2
    y = gemm_ref_f64(x_bits, codes, scales, g)
    return silu_f64(y[:, :n]) * y[:, n:]


def residual_ref_f64(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, g: int,
                     r_bits: np.ndarray, gate_bits: np.ndarray) -> np.ndarray:
    """Y[m, n] = R[m, n] + gate[n] * (X @ W.T)[m, n] in fp64, R and gate given as bf16 bit
    patterns (reading R7)."""
    y = gemm_ref_f64(x_bits, codes, scales, g)
    r = bf16_bits_to_f64(r_bits)
    gt = bf16_bits_to_f64(gate_bits)
    if r.shape != y.shape or gt.shape != (y.shape[1],):
        raise ValueError("residual must be [M, N] and gate [N]")
    return r + gt[None, :] * y


# ----------------------------------------------------------------------------------------
# Affine 4-bit groups (reading R10)
# ----------------------------------------------------------------------------------------

def pack_u4(levels: np.ndarray) -> Tuple[np.ndarray, int]:
    """Unsigned 4-bit levels [N, K] (0 .. 15) -> (uint32 words [N, K/8], number of invalid
    levels).  Level k of a row sits at bits 4*(k % 8) of word k // 8; levels outside 0 .. 15
    pack as 0 and are counted."""
    q = np.asarray(levels, dtype=np.int64)
    if q.ndim != 2 or q.shape[1] % 8:
        raise ValueError("levels must be [N, K] with K a multiple of 8")
    N, K = q.shape
    ok = (q >= 0) & (q <= 15)
    field = np.where(ok, q, 0).astype(np.uint32).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        words |= field[:, :, i] << np.uint32(4 * i)
    return words, int(np.count_nonzero(~ok))


def unpack_u4(words: np.ndarray, K: int) -> np.ndarray:
    """uint32 words [N, K/8] -> unsigned levels [N, K] (uint8, 0 .. 15)."""
    w = np.asarray(words, dtype=np.uint32)
    N = w.shape[0]
    if w.shape[1] * 8 != K:
        raise ValueError("words do not hold K levels per row")
    out = np.zeros((N, w.shape[1], 8), dtype=np.uint8)
    for i in range(8):
        out[:, :, i] = ((w >> np.uint32(4 * i)) & np.uint32(15)).astype(np.uint8)
    return out.reshape(N, K)


def dequant_affine_f64(levels: np.ndarray, scales: np.ndarray, biases: np.ndarray, g: int) -> np.ndarray:
    """W[n, k] = q[n, k] * S[n, k // g] + B[n, k // g] in fp64.  Exact: q * s has at most
    4 + 11 significant bits and adding the fp16 bias needs far fewer than fp64's 53."""
    q = np.asarray(levels).astype(np.float64)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    b = np.asarray(biases, dtype=np.float16).astype(np.float64)
    N, K = q.shape
    if K % g or s.shape != (N, K // g) or b.shape != (N, K // g):
        raise ValueError("scales and biases must be [N, K // g]")
    return q * np.repeat(s, g, axis=1) + np.repeat(b, g, axis=1)


def gemm_affine_ref_f64(x_bits: np.ndarray, levels: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                        g: int) -> np.ndarray:
    """Y = X @ dequant_affine(W).T in fp64: dequantise to dense, then an ordinary matmul."""
    xd = bf16_bits_to_f64(x_bits)
    wd = dequant_affine_f64(levels, scales, biases, g)
    if xd.shape[1] != wd.shape[1]:
        raise ValueError("X and W disagree on K")
    return xd @ wd.T


def gemm_affine_fsum_element(x_bits: np.ndarray, levels: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                             g: int, m: int, n: int) -> float:
    """One affine output element as the correctly rounded sum (math.fsum) of its exact terms
    x * q * s and x * b."""
    x = bf16_bits_to_f64(np.asarray(x_bits)[m])
    q = np.asarray(levels)[n]
    s = np.asarray(scales, dtype=np.float16)[n].astype(np.float64)
    b = np.asarray(biases, dtype=np.float16)[n].astype(np.float64)
    terms = []
    for k in range(q.shape[0]):
        terms.append(float(x[k]) * int(q[k]) * float(s[k // g]))
        terms.append(float(x[k]) * float(b[k // g]))
    return math.fsum(terms)


# ----------------------------------------------------------------------------------------
# Acceptance
# ----------------------------------------------------------------------------------------

def check_tolerance(y: np.ndarray, yref: np.ndarray, rel_frob_tol: float = REL_FROB_TOL,
                    elem_tol: float = ELEM_TOL) -> Dict[str, float]:
    """Accept y iff ||y - yref||_F / ||yref||_F <= rel_frob_tol and, for every element,
    |y - yref| <= elem_tol * (|yref| + 1).  `y` may be bf16 bit patterns (uint16) or
    floats."""
    y = np.asarray(y)
    yf = bf16_bits_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    err = yf - yref
    nref = float(np.linalg.norm(yref))
    rel = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    ratio = np.abs(err) / (np.abs(yref) + 1.0)
    max_ratio = float(ratio.max()) if ratio.size else 0.0
    finite = bool(np.all(np.isfinite(yf)))
    ok = finite and rel <= rel_frob_tol and max_ratio <= elem_tol
    return {"ok": ok, "rel_frob": rel, "max_ratio": max_ratio, "finite": finite}
