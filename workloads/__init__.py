"""Seeded synthetic inputs for the packed low-bit weight GEMM.

This module only draws random inputs: bf16 activations, int8 weight codes and
fp16 group scales.  It holds none of the GEMM's arithmetic (no packing, no
unpacking, no dequantisation, no products), so that the oracle and the HIP path
can both be fed from it without sharing any of the method.

Recipe (one reading per quantity; the pages give shapes and formats but no
input distributions):

* X[m, k]   : fp32 standard normal, rounded to bf16 with round-to-nearest-even.
              Stands in for FLUX.2 Klein token activations (image tokens
              (H/16)*(W/16) plus 512 text tokens).
* codes     : ternary {-1, 0, +1} with probabilities {0.25, 0.5, 0.25}, or binary
              {-1, +1} with probability 0.5 each, i.i.d.
* S[n, grp] : uniform on [0.005, 0.05], rounded to fp16 (all normal numbers).
* streams   : every tensor has its own PCG64 stream seeded by
              SeedSequence([seed, config_id, tensor_id]).

Shapes follow the FLUX.2 Klein 4B MMDiT linears described on the
"bonsai-image-binary-4B-gemlite-1bit" model card (section "Model Overview": 25
MMDiT blocks, 5 double-stream + 20 single-stream, all matmul-heavy linears
quantised), with hidden size 3072.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

TERNARY = 2
BINARY = 1
INT4 = 4


def rng_for(seed: int, config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, tensor_id])))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (finite inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def gen_x(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """bf16 bit patterns, shape [M, K], dtype uint16."""
    return _f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


_TERNARY_FROM_2BITS = np.array([-1, 0, 0, 1], dtype=np.int8)


def gen_codes(rng: np.random.Generator, N: int, K: int, bits: int) -> np.ndarray:
    """int8 codes, shape [N, K]: ternary P(-1)=P(+1)=1/4, P(0)=1/2; binary P(+-1)=1/2;
    4-bit uniform on the integers -8 .. 7."""
    if bits == TERNARY:
        u = rng.integers(0, 4, size=(N, K), dtype=np.uint8)
        return _TERNARY_FROM_2BITS[u]
    if bits == BINARY:
        u = rng.integers(0, 2, size=(N, K), dtype=np.int8)
        return (u * np.int8(2) - np.int8(1)).astype(np.int8)
    if bits == INT4:
        return rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    raise ValueError(f"bits must be 1, 2 or 4, got {bits}")


def gen_levels(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Unsigned 4-bit levels of affine groups, shape [N, K], uniform on 0 .. 15 (int8)."""
    return rng.integers(0, 16, size=(N, K), dtype=np.int8)


def gen_biases(rng: np.random.Generator, N: int, K: int, g: int) -> np.ndarray:
    """fp16 group biases of affine groups, shape [N, K // g], uniform on [-0.45, -0.03]: the
    range of -z * s for zero points z in [6, 9] and the scales of gen_scales, drawn
    independently of the scales."""
    if K % g:
        raise ValueError("K must be a multiple of g")
    return rng.uniform(-0.45, -0.03, size=(N, K // g)).astype(np.float16)


def gen_scales(rng: np.random.Generator, N: int, K: int, g: int) -> np.ndarray:
    """fp16 group scales, shape [N, K // g], uniform on [0.005, 0.05]."""
    if K % g:
        raise ValueError("K must be a multiple of g")
    return rng.uniform(0.005, 0.05, size=(N, K // g)).astype(np.float16)


@dataclasses.dataclass(frozen=True)
class Problem:
    """One GEMM Y[M,N] = X[M,K] . dequant(W)[N,K]^T of a workload."""
    name: str
    M: int
    N: int
    K: int
    bits: int = TERNARY
    g: int = 64
    config_id: int = 0
    tensor_id: int = 0
    affine: bool = False   # 4-bit affine groups: levels 0 .. 15 with a scale and a bias per group

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes: X + packed W + fp16 scales + Y."""
        groups = 2 if self.affine else 1  # fp16 scales (and biases)
        return (2 * self.M * self.K + self.N * self.K * self.bits // 8
                + 2 * groups * self.N * (self.K // self.g) + 2 * self.M * self.N)


@dataclasses.dataclass
class Inputs:
    x: np.ndarray       # uint16 bf16 bits [M, K]
    codes: np.ndarray   # int8 [N, K] (affine problems: the unsigned levels 0 .. 15)
    scales: np.ndarray  # float16 [N, K // g]
    biases: np.ndarray | None = None  # float16 [N, K // g], affine problems only


def make_inputs(p: Problem, seed: int = 0, x_tensor_id: int | None = None) -> Inputs:
    """Draw the inputs of one problem.  X uses tensor id `x_tensor_id` (default: the
    problem's id * 3), codes id*3+1, scales id*3+2, so that problems that share an
    activation can say so."""
    base = p.tensor_id * 3
    xid = base if x_tensor_id is None else x_tensor_id
    x = gen_x(rng_for(seed, p.config_id, xid), p.M, p.K)
    if p.affine:
        levels = gen_levels(rng_for(seed, p.config_id, base + 1), p.N, p.K)
        scales = gen_scales(rng_for(seed, p.config_id, base + 2), p.N, p.K, p.g)
        biases = gen_biases(rng_for(seed, p.config_id, 100000 + p.tensor_id), p.N, p.K, p.g)
        return Inputs(x, levels, scales, biases)
    codes = gen_codes(rng_for(seed, p.config_id, base + 1), p.N, p.K, p.bits)
    scales = gen_scales(rng_for(seed, p.config_id, base + 2), p.N, p.K, p.g)
    return Inputs(x, codes, scales)


# --------------------------------------------------------------------------------------
# Workloads.  Hidden size 3072; QKV fused (3 x 3072); SwiGLU MLP-in 2 x 9216; single-stream
# fused linear 3 x 3072 + 2 x 9216 = 27648 and its output 3072 + 9216 = 12288 -> 3072.
# M = (H/16)(W/16) image tokens + 512 text tokens.
# --------------------------------------------------------------------------------------

TINY = [Problem("tiny_ternary", 64, 256, 256, TERNARY, 64, 0, 0)]

_BLOCK_SHAPES = [("proj", 3072, 3072), ("qkv", 9216, 3072), ("mlp_in", 18432, 3072), ("mlp_out", 3072, 9216)]

RES512_TERNARY = [Problem(f"m1536_{n}", 1536, N, K, TERNARY, 64, 1, i)
                  for i, (n, N, K) in enumerate(_BLOCK_SHAPES)]
RES512_BINARY = [Problem(f"m1536_{n}_bin", 1536, N, K, BINARY, 64, 2, i)
                 for i, (n, N, K) in enumerate(_BLOCK_SHAPES)]
RES1024_TERNARY = [Problem(f"m4608_{n}", 4608, N, K, TERNARY, 64, 3, i)
                   for i, (n, N, K) in enumerate(_BLOCK_SHAPES + [("single_out", 3072, 12288)])]
# the binary model card's own format: 1-bit codes with one fp16 scale per 128 weights
# ("bonsai-image-binary-4B-gemlite-1bit" model card, "Binary Weight Representation: 1-bit g128")
RES1024_BINARY_G128 = [Problem(f"m4608_{n}_bin128", 4608, N, K, BINARY, 128, 5, i)
                       for i, (n, N, K) in enumerate(_BLOCK_SHAPES + [("single_out", 3072, 12288)])]


def denoise_step_sweep(M_img: int = 4096, M_txt: int = 512, bits: int = TERNARY, g: int = 64,
                       skinny_m: int | None = None) -> List[Problem]:
    """The 80 quantised GEMMs of one FLUX.2 Klein 4B denoise step at 1024x1024.

    Double-stream blocks run the image stream (M_img tokens) and the text stream (M_txt
    tokens) with separate weights: QKV 3072->9216, proj 3072->3072, MLP-in 3072->18432,
    MLP-out 9216->3072.  Single-stream blocks run all M_img + M_txt tokens through the
    fused 3072->27648 linear and the 12288->3072 output linear.  With `skinny_m`, every
    GEMM runs at that M instead (the decode-like skinny variant)."""
    probs: List[Problem] = []
    tid = 0
    for b in range(5):
        for stream, m in (("img", M_img), ("txt", M_txt)):
            for n, N, K in (("qkv", 9216, 3072), ("proj", 3072, 3072),
                            ("mlp_in", 18432, 3072), ("mlp_out", 3072, 9216)):
                probs.append(Problem(f"d{b}_{stream}_{n}", skinny_m or m, N, K, bits, g, 4, tid))
                tid += 1
    for b in range(20):
        for n, N, K in (("fused", 27648, 3072), ("out", 3072, 12288)):
            probs.append(Problem(f"s{b}_{n}", skinny_m or (M_img + M_txt), N, K, bits, g, 4, tid))
            tid += 1
    return probs


def step_groups(probs: List[Problem]) -> List[List[int]]:
    """Indices of `probs` (a denoise_step_sweep list) in launch order, grouped the way the
    model allows: a double-stream block's image and text linear of one kind are independent
    and go together; everything else is sequential and goes alone."""
    groups: List[List[int]] = []
    pending: dict = {}
    for i, p in enumerate(probs):
        parts = p.name.split("_", 2)
        if p.name.startswith("d") and len(parts) == 3:
            key = (parts[0], parts[2])
            if key in pending:
                groups[pending.pop(key)].append(i)
                continue
            pending[key] = len(groups)
        groups.append([i])
    # within a block: qkv, proj, mlp_in, mlp_out pairs in that order
    return groups


CONFIGS = {
    "tiny": TINY,
    "res512_ternary": RES512_TERNARY,
    "res512_binary": RES512_BINARY,
    "res1024_ternary": RES1024_TERNARY,
    "res1024_binary_g128": RES1024_BINARY_G128,
}


def distinct_shapes(probs: List[Problem]) -> List[Tuple[Tuple[int, int, int, int, int], int]]:
    """[(M, N, K, bits, g), count] in first-seen order."""
    seen: dict = {}
    for p in probs:
        key = (p.M, p.N, p.K, p.bits, p.g)
        seen[key] = seen.get(key, 0) + 1
    return list(seen.items())
