"""Helpers shared by the GPU tests: move seeded numpy inputs to the device and run the
library through its C-ABI binding.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np

import binary_bit_gemm_amd as lb


def torch():
    import torch as t
    return t


def dev_x(x_bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(t.bfloat16).cuda()


def dev_codes(codes: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(codes, dtype=np.int8)).cuda()


def dev_scales(s: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(s, dtype=np.float16)).cuda()


def dev_words(words_u32: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(words_u32, dtype=np.uint32).view(np.int32)).cuda()


def host_bits(y) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    t = torch()
    return y.view(t.int16).cpu().numpy().view(np.uint16)


def host_words(w) -> np.ndarray:
    return w.cpu().numpy().view(np.uint32)


def run_gemm(inp, g: int, bits: int):
    """Pack codes on the GPU, run lowbit_gemm, return (Y bits uint16 [M,N], packed words)."""
    x = dev_x(inp.x)
    words, bad = lb.pack(dev_codes(inp.codes), bits)
    assert bad == 0
    s = dev_scales(inp.scales)
    y = lb.gemm(x, words, s, g, bits)
    torch().cuda.synchronize()
    return host_bits(y), words
