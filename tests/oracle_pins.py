"""Pins that tie the oracle to facts outside itself.

Each pin takes the oracle as an object `o` exposing pack / unpack / dequant_f64 /
gemm_ref_f64 / gemm_fsum_element, so that tests/test_oracle.py can run every pin on the
real oracle (all must pass) and on copies with a planted mistake (some pin must fail).
None of these re-types the oracle's formulas: the expected values come from hand-worked
golden words, bit strings built a different way, math.fsum of exact products,
closed-form statistics, exact algebraic identities, or a library matmul.
"""
from __future__ import annotations

import math
import os
from types import SimpleNamespace

import numpy as np

from workloads import gen_codes, gen_scales, gen_x, rng_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_words.txt")


def load_golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            b, name, codes, word = [s.strip() for s in line.split("|")]
            rows.append((int(b), name, np.array([int(v) for v in codes.split(",")], dtype=np.int8),
                         int(word, 16)))
    return rows


def real_oracle():
    import oracle
    return SimpleNamespace(pack=oracle.pack, unpack=oracle.unpack, dequant_f64=oracle.dequant_f64,
                           gemm_ref_f64=oracle.gemm_ref_f64, gemm_fsum_element=oracle.gemm_fsum_element,
                           bf16_bits_to_f64=oracle.bf16_bits_to_f64, silu_f64=oracle.silu_f64,
                           swiglu_ref_f64=oracle.swiglu_ref_f64, residual_ref_f64=oracle.residual_ref_f64,
                           gemlite_u8t_decode=oracle.gemlite_u8t_decode, gemlite_u8t_encode=oracle.gemlite_u8t_encode,
                           mlx_u32_decode=oracle.mlx_u32_decode, mlx_u32_encode=oracle.mlx_u32_encode,
                           gemlite_binary_decode=oracle.gemlite_binary_decode,
                           gemlite_binary_encode=oracle.gemlite_binary_encode,
                           pack_u4=oracle.pack_u4, unpack_u4=oracle.unpack_u4,
                           dequant_affine_f64=oracle.dequant_affine_f64,
                           gemm_affine_ref_f64=oracle.gemm_affine_ref_f64,
                           gemm_affine_fsum_element=oracle.gemm_affine_fsum_element)


# ----------------------------------------------------------------------------------------

def pin_golden_words(o):
    """Packing and unpacking reproduce the hand-worked golden words."""
    for bits, name, codes, word in load_golden():
        w, bad = o.pack(codes[None, :], bits)
        assert bad == 0, name
        assert w.shape == (1, 1) and int(w[0, 0]) == word, f"{name}: {int(w[0, 0]):#010x} != {word:#010x}"
        back = o.unpack(np.array([[word]], dtype=np.uint32), codes.size, bits)
        assert np.array_equal(back[0], codes), name


def pin_bitstring(o, seed=11):
    """Words equal integers parsed from bit strings written most-significant field first."""
    rng = np.random.default_rng(seed)
    for bits in (2, 1):
        per = 32 // bits
        codes = gen_codes(rng, 5, 4 * per, bits)
        w, _ = o.pack(codes, bits)
        for n in range(codes.shape[0]):
            for j in range(4):
                chunk = codes[n, j * per:(j + 1) * per]
                if bits == 2:
                    fields = ["01" if c == 1 else "10" if c == -1 else "00" for c in chunk]
                else:
                    fields = ["1" if c == 1 else "0" for c in chunk]
                expect = int("".join(reversed(fields)), 2)
                assert int(w[n, j]) == expect


def pin_group_blocks(o):
    """Scale group membership: with X = 1 on exactly one run of g consecutive k and all
    codes +1, Y[m, n] = g * (scale of that run).  The expected value picks the scale by
    the run's position, not by evaluating k // g."""
    K, g, N = 256, 64, 3
    scales = (np.arange(N * (K // g)).reshape(N, K // g) + 1).astype(np.float16) / np.float16(16)
    codes = np.ones((N, K), dtype=np.int8)
    for run in range(K // g):
        x = np.zeros((1, K), dtype=np.uint16)
        x[0, run * g:(run + 1) * g] = 0x3F80  # bf16 1.0
        y = o.gemm_ref_f64(x, codes, scales, g)
        for n in range(N):
            assert y[0, n] == g * float(scales[n, run]), (run, n)


def pin_one_hot(o):
    """Exactly one nonzero code c[n0, k0] = -1: Y[:, n0] = -S[n0, grp] * X[:, k0] where grp is
    the run of g consecutive k holding k0 (worked out by hand below), and every other
    column is exactly 0.  The square case catches a transposed decode."""
    rng = rng_for(5, 99, 0)
    for (M, N, K, g, cases) in ((4, 8, 128, 32, ((0, 0, 0), (3, 31, 0), (5, 32, 1), (7, 127, 3), (2, 77, 2))),
                                (3, 64, 64, 32, ((1, 40, 1), (50, 3, 0)))):
        x = gen_x(rng, M, K)
        s = gen_scales(rng, N, K, g)
        xf = o.bf16_bits_to_f64(x)
        for (n0, k0, grp) in cases:
            c = np.zeros((N, K), dtype=np.int8)
            c[n0, k0] = -1
            w, _ = o.pack(c, 2)
            y = o.gemm_ref_f64(x, o.unpack(w, K, 2), s, g)
            assert np.array_equal(y[:, n0], -float(s[n0, grp]) * xf[:, k0]), (n0, k0)
            assert not np.any(np.delete(y, n0, axis=1)), (n0, k0)


def pin_unpack_unused_field(o):
    """The ternary field 11 (never written by the packer) decodes to 0; a binary word of
    all ones decodes to all +1."""
    w = np.full((2, 3), 0xFFFFFFFF, dtype=np.uint32)
    assert not np.any(o.unpack(w, 48, 2))
    assert np.all(o.unpack(w, 96, 1) == 1)


def pin_fsum(o, M=64, N=256, K=256, g=64, bits=2, seed=0):
    """fp64 dgemm result within a few ulps of the correctly rounded exact sum."""
    x = gen_x(rng_for(seed, 0, 0), M, K)
    c = gen_codes(rng_for(seed, 0, 1), N, K, bits)
    s = gen_scales(rng_for(seed, 0, 2), N, K, g)
    y = o.gemm_ref_f64(x, c, s, g)
    xf = o.bf16_bits_to_f64(x)
    sf = np.repeat(s.astype(np.float64), g, axis=1)
    for m in range(M):
        for n in range(N):
            terms = [float(a) * int(b) * float(t) for a, b, t in zip(xf[m], c[n], sf[n])]
            exact = math.fsum(terms)
            bound = 4 * K * np.finfo(np.float64).eps * math.fsum(abs(t) for t in terms)
            assert abs(y[m, n] - exact) <= bound, (m, n, y[m, n], exact)
    # and the single-element brute force agrees bit for bit with the fsum above
    for (m, n) in ((0, 0), (M - 1, N - 1), (M // 3, N // 2 + 1)):
        e = o.gemm_fsum_element(x, c, s, g, m, n)
        terms = [float(a) * int(b) * float(t) for a, b, t in zip(xf[m], c[n], sf[n])]
        assert e == math.fsum(terms)


def pin_statistics(o, bits=2, M=128, N=256, K=3072, g=64, seed=3):
    """E[y] = 0 and Var(y) = K * P(c != 0) * E[s^2] * E[x^2] for independent inputs with
    x ~ N(0,1), s ~ U[0.005, 0.05] (E[s^2] = (a^2 + ab + b^2)/3 = 9.25e-4)."""
    x = gen_x(rng_for(seed, 7, 0), M, K)
    c = gen_codes(rng_for(seed, 7, 1), N, K, bits)
    s = gen_scales(rng_for(seed, 7, 2), N, K, g)
    y = o.gemm_ref_f64(x, c, s, g)
    p_nz = 0.5 if bits == 2 else 1.0
    var = K * p_nz * (0.005 ** 2 + 0.005 * 0.05 + 0.05 ** 2) / 3.0
    assert abs(y.mean()) < 0.05 * math.sqrt(var)
    assert abs(y.var() / var - 1.0) < 0.06, (y.var(), var)


def pin_linearity(o, seed=4):
    """Exact identities: Y(2^e S) = 2^e Y(S), Y(-X) = -Y(X), Y(-c) = -Y(c)."""
    M, N, K, g = 16, 32, 256, 64
    x = gen_x(rng_for(seed, 8, 0), M, K)
    c = gen_codes(rng_for(seed, 8, 1), N, K, 2)
    s = gen_scales(rng_for(seed, 8, 2), N, K, g)
    y = o.gemm_ref_f64(x, c, s, g)
    y2 = o.gemm_ref_f64(x, c, (s.astype(np.float32) * 4).astype(np.float16), g)
    assert np.array_equal(y2, 4 * y)
    assert np.array_equal(o.gemm_ref_f64(x ^ np.uint16(0x8000), c, s, g), -y)
    assert np.array_equal(o.gemm_ref_f64(x, -c, s, g), -y)
    zero = o.gemm_ref_f64(x, np.zeros_like(c), s, g)
    assert not np.any(zero)


def pin_library_matmul(o, seed=6):
    """With every scale 1, dequant(W) is the codes themselves and Y is a plain matmul,
    here computed by torch's CPU matmul in float64."""
    import torch
    M, N, K, g = 32, 48, 192, 64
    x = gen_x(rng_for(seed, 9, 0), M, K)
    c = gen_codes(rng_for(seed, 9, 1), N, K, 2)
    ones = np.ones((N, K // g), dtype=np.float16)
    y = o.gemm_ref_f64(x, c, ones, g)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    ref = torch.matmul(xt, torch.from_numpy(c.astype(np.float64)).T).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def pin_binary_is_ternary_without_zeros(o, seed=8):
    """The same {-1,+1} codes packed as binary and as ternary decode to the same codes and
    give identical Y."""
    M, N, K, g = 8, 16, 128, 64
    x = gen_x(rng_for(seed, 10, 0), M, K)
    c = gen_codes(rng_for(seed, 10, 1), N, K, 1)
    s = gen_scales(rng_for(seed, 10, 2), N, K, g)
    wb, _ = o.pack(c, 1)
    wt, _ = o.pack(c, 2)
    cb = o.unpack(wb, K, 1)
    ct = o.unpack(wt, K, 2)
    assert np.array_equal(cb, c) and np.array_equal(ct, c)
    assert np.array_equal(o.gemm_ref_f64(x, cb, s, g), o.gemm_ref_f64(x, ct, s, g))


ALL_PINS = [pin_golden_words, pin_bitstring, pin_unpack_unused_field, pin_group_blocks, pin_one_hot, pin_fsum,
            pin_statistics, pin_linearity, pin_library_matmul, pin_binary_is_ternary_without_zeros]


# ----------------------------------------------------------------------------------------
# SwiGLU (silu(gate) * up over the [gate | up] halves of the MLP-in weights)
# ----------------------------------------------------------------------------------------

# logistic function values sigma(t) = 1 / (1 + e^-t) and sigma(-t), to 16 significant digits
_SIGMOID = {1.0: (0.7310585786300049, 0.2689414213699951), 2.0: (0.8807970779778823, 0.1192029220221176),
            4.0: (0.9820137900379085, 0.01798620996209156), 20.0: (0.9999999979388463, 2.061153618190204e-09)}


def pin_silu_values(o):
    """silu(t) = t * sigma(t) and silu(-t) = -t * sigma(-t) at points where sigma is tabulated above."""
    for t, (sp, sn) in _SIGMOID.items():
        got = o.silu_f64(np.array([t, -t]))
        assert abs(got[0] - t * sp) <= 1e-15 * t, (t, got[0])
        assert abs(got[1] + t * sn) <= 1e-14 * t * sn, (t, got[1])
    assert o.silu_f64(np.array([0.0]))[0] == 0.0


def pin_silu_identities(o, seed=21):
    """silu(-a) = silu(a) - a for all a; silu(a) -> a for large a; no overflow for very negative a."""
    a = np.random.default_rng(seed).normal(0.0, 6.0, 4096)
    lhs, rhs = o.silu_f64(-a), o.silu_f64(a) - a
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    big = o.silu_f64(np.array([50.0, 700.0]))
    assert abs(big[0] - 50.0) <= 1e-12 and big[1] == 700.0
    tiny = o.silu_f64(np.array([-800.0, -1e4]))
    assert np.all(np.isfinite(tiny)) and np.all(tiny <= 0.0) and np.all(np.abs(tiny) < 1e-300)


def pin_swiglu_fsum(o, seed=23):
    """Each element equals silu(gate) * up with gate and up the correctly rounded sums of their exact
    products (math.fsum) and silu from the math library's exp."""
    M, N, K, g = 6, 32, 192, 64
    x = gen_x(rng_for(seed, 11, 0), M, K)
    c = gen_codes(rng_for(seed, 11, 1), 2 * N, K, 2)
    sc = gen_scales(rng_for(seed, 11, 2), 2 * N, K, g)
    y = o.swiglu_ref_f64(x, c, sc, g)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            gt = o.gemm_fsum_element(x, c, sc, g, m, n)
            up = o.gemm_fsum_element(x, c, sc, g, m, N + n)
            want = gt / (1.0 + math.exp(-gt)) * up
            assert abs(y[m, n] - want) <= 1e-12 * (abs(want) + 1e-30) + 1e-15, (m, n, y[m, n], want)


def pin_swiglu_halves(o, seed=25):
    """Gate rows first: the result is silu(Y of rows [0, N)) * (Y of rows [N, 2N)) of the plain
    GEMM on each half alone, and swapping the halves changes it."""
    M, N, K, g = 8, 48, 256, 64
    x = gen_x(rng_for(seed, 12, 0), M, K)
    c = gen_codes(rng_for(seed, 12, 1), 2 * N, K, 2)
    sc = gen_scales(rng_for(seed, 12, 2), 2 * N, K, g)
    gt = o.gemm_ref_f64(x, c[:N], sc[:N], g)
    up = o.gemm_ref_f64(x, c[N:], sc[N:], g)
    y = o.swiglu_ref_f64(x, c, sc, g)
    assert np.allclose(y, gt / (1.0 + np.exp(-gt)) * up, rtol=1e-12, atol=1e-14)
    swapped = o.swiglu_ref_f64(x, np.concatenate([c[N:], c[:N]]), np.concatenate([sc[N:], sc[:N]]), g)
    assert not np.allclose(y, swapped, rtol=1e-3, atol=1e-3)


SWIGLU_PINS = [pin_silu_values, pin_silu_identities, pin_swiglu_fsum, pin_swiglu_halves]


# ----------------------------------------------------------------------------------------
# Gated residual (Y = R + gate[n] * (X . W^T))
# ----------------------------------------------------------------------------------------

def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """Exact bf16 bit patterns of values that bf16 holds exactly (the top half of their fp32 bits)."""
    f = np.asarray(v, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64)), "not exact in fp32"
    b = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << np.uint32(16)).view(np.float32), f), "not exact in bf16"
    return b


def _residual_case(seed, M=6, N=32, K=192, g=64):
    x = gen_x(rng_for(seed, 13, 0), M, K)
    c = gen_codes(rng_for(seed, 13, 1), N, K, 2)
    sc = gen_scales(rng_for(seed, 13, 2), N, K, g)
    r = gen_x(rng_for(seed, 13, 3), M, N)              # bf16 bit patterns
    gt = gen_x(rng_for(seed, 13, 4), 1, N)[0]
    return x, c, sc, g, r, gt


def pin_residual_special_gates(o, seed=31):
    """gate = 0 gives the residual exactly; residual = 0 and gate = 1 give the plain GEMM exactly."""
    x, c, sc, g, r, _ = _residual_case(seed)
    N = c.shape[0]
    zero = _bf16_bits(np.zeros(N))
    one = _bf16_bits(np.ones(N))
    assert np.array_equal(o.residual_ref_f64(x, c, sc, g, r, zero), o.bf16_bits_to_f64(r))
    rz = _bf16_bits(np.zeros(r.shape))
    assert np.array_equal(o.residual_ref_f64(x, c, sc, g, rz, one), o.gemm_ref_f64(x, c, sc, g))


def pin_residual_fsum(o, seed=33):
    """Each element equals R + gate * (the correctly rounded sum of the exact products), R and gate
    read from their bf16 bit patterns by hand (sign, exponent, mantissa)."""
    x, c, sc, g, r, gt = _residual_case(seed)
    y = o.residual_ref_f64(x, c, sc, g, r, gt)

    def bf16(b):
        b = int(b)
        sgn = -1.0 if b >> 15 else 1.0
        e, m = (b >> 7) & 0xFF, b & 0x7F
        return sgn * (m / 128.0) * 2.0 ** -126 if e == 0 else sgn * (1 + m / 128.0) * 2.0 ** (e - 127)

    for m in range(y.shape[0]):
        for n in range(y.shape[1]):
            want = bf16(r[m, n]) + bf16(gt[n]) * o.gemm_fsum_element(x, c, sc, g, m, n)
            assert abs(y[m, n] - want) <= 1e-13 * (abs(want) + 1.0), (m, n, y[m, n], want)


def pin_residual_gate_linearity(o, seed=35):
    """Doubling the gate doubles Y - R exactly; the gate acts per output column (a one-hot gate
    leaves every other column equal to R)."""
    x, c, sc, g, r, gt = _residual_case(seed)
    rf = o.bf16_bits_to_f64(r)
    y1 = o.residual_ref_f64(x, c, sc, g, r, gt)
    y2 = o.residual_ref_f64(x, c, sc, g, r, _bf16_bits(2.0 * o.bf16_bits_to_f64(gt)))
    assert np.array_equal(y2 - rf, 2.0 * (y1 - rf))
    N = c.shape[0]
    hot = np.zeros(N)
    hot[5] = 1.0
    yh = o.residual_ref_f64(x, c, sc, g, r, _bf16_bits(hot))
    others = np.arange(N) != 5
    assert np.array_equal(yh[:, others], rf[:, others])
    assert not np.array_equal(yh[:, 5], rf[:, 5])


RESIDUAL_PINS = [pin_residual_special_gates, pin_residual_fsum, pin_residual_gate_linearity]


# ----------------------------------------------------------------------------------------
# Importers (GemLite transposed uint8, MLX uint32 rows; unsigned levels q, code q - zero)

def pin_import_golden(o):
    """Hand-worked bytes and words of the two source layouts (levels: 0 -> 00, 1 -> 01,
    2 -> 10, least significant field first; zero = 1 maps codes -1, 0, +1 to levels 0, 1, 2)."""
    z = np.zeros((16, 16), dtype=np.int8)
    assert np.all(o.gemlite_u8t_encode(z) == 0x55)            # level 1 in all four fields
    assert np.all(o.gemlite_u8t_encode(z + 1) == 0xAA)        # level 2
    assert np.all(o.gemlite_u8t_encode(z - 1) == 0x00)        # level 0
    one = z.copy()
    one[2, 5] = -1                                            # row 2, k = 5: byte (1, 2), field 1
    b = o.gemlite_u8t_encode(one)
    assert b.shape == (4, 16) and b[1, 2] == 0x51 and np.count_nonzero(b != 0x55) == 1
    codes, bad = o.gemlite_u8t_decode(b, 16, 16)
    assert bad == 0 and np.array_equal(codes, one)
    # a square source buffer (K/4 == N == 16): code (n = 0, k = 63) sits in byte (15, 0),
    # field 3; read in the direct orientation it would land in row 15
    sq = np.full((16, 16), 0x55, dtype=np.uint8)
    sq[15, 0] = 0x95                                          # 10 01 01 01
    codes, bad = o.gemlite_u8t_decode(sq, 16, 64)
    assert bad == 0 and codes[0, 63] == 1 and np.count_nonzero(codes) == 1
    # MLX rows
    z = np.zeros((16, 32), dtype=np.int8)
    assert np.all(o.mlx_u32_encode(z) == 0x55555555)
    one = z.copy()
    one[0, 0] = 1
    one[1, 31] = -1                                           # word (1, 1), field 15 -> level 0
    w = o.mlx_u32_encode(one)
    assert w[0, 0] == 0x55555556 and w[1, 1] == 0x15555555 and np.count_nonzero(w != 0x55555555) == 2
    codes, bad = o.mlx_u32_decode(w, 16, 32)
    assert bad == 0 and np.array_equal(codes, one)
    # level 3 is no ternary code at zero = 1; at zero = 3 levels 0 .. 2 are the invalid ones
    codes, bad = o.gemlite_u8t_decode(np.full((4, 16), 0xFF, dtype=np.uint8), 16, 16)
    assert bad == 256 and not codes.any()
    codes, bad = o.gemlite_u8t_decode(np.full((4, 16), 0xFF, dtype=np.uint8), 16, 16, zero=3)
    assert bad == 0 and not codes.any()
    codes, bad = o.mlx_u32_decode(np.full((16, 1), 0x00000001, dtype=np.uint32), 16, 16, zero=0)
    assert bad == 0 and np.all(codes[:, 0] == 1) and not codes[:, 1:].any()
    codes, bad = o.mlx_u32_decode(np.full((16, 1), 0x00000001, dtype=np.uint32), 16, 16, zero=3)
    assert bad == 16 * 16 and not codes.any()


def pin_import_other_routes(o, seed=41):
    """The decoders against routes written differently: the library's field of code q - 1 is
    (q + 2) mod 3 (levels 0, 1, 2 -> fields 10, 00, 01), read from base-4 digits of Python
    integers; GemLite bytes through numpy's little-endian unpackbits and a transpose."""
    rng = np.random.default_rng(seed)
    N, K = 32, 96
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    w = o.mlx_u32_encode(codes)
    got, bad = o.mlx_u32_decode(w, N, K)
    assert bad == 0 and np.array_equal(got, codes)
    packed, _ = o.pack(got, 2)
    for n in range(N):
        for j in range(K // 16):
            v, expect = int(w[n, j]), 0
            for i in range(16):
                v, q = divmod(v, 4)
                expect += ((q + 2) % 3) * 4 ** i
            assert int(packed[n, j]) == expect
    b = o.gemlite_u8t_encode(codes)
    bits = np.unpackbits(b[:, :, None], axis=2, bitorder="little")          # [K/4, N, 8]
    levels = (bits[:, :, 0::2] + 2 * bits[:, :, 1::2]).astype(np.int64)     # [K/4, N, 4]
    direct = levels.transpose(0, 2, 1).reshape(K, N).T - 1
    assert np.array_equal(direct, codes)
    got, bad = o.gemlite_u8t_decode(b, N, K)
    assert bad == 0 and np.array_equal(got, codes)


def pin_import_layouts_agree(o, seed=43):
    """The same weight through either layout decodes to the same codes, at every zero point
    whose levels fit in 2 bits."""
    rng = np.random.default_rng(seed)
    N, K = 48, 64
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    for zero in (1, 2):
        a, ba = o.gemlite_u8t_decode(o.gemlite_u8t_encode(codes, zero), N, K, zero)
        m, bm = o.mlx_u32_decode(o.mlx_u32_encode(codes, zero), N, K, zero)
        assert ba == bm == 0 and np.array_equal(a, codes) and np.array_equal(m, codes)


def pin_import_binary(o, seed=45):
    """GemLite 1-bit bytes: hand-worked values (all +1 -> 0xFF, all -1 -> 0x00, code (2, 5) = +1
    among -1 -> byte (0, 2) = 0x20; a square buffer, K/8 = N = 16, with code (0, 127) = +1 in
    byte (15, 0) = 0x80), and random codes through numpy's little-endian unpackbits and a
    transpose, then through the library's own binary words."""
    z = -np.ones((16, 16), dtype=np.int8)
    assert np.all(o.gemlite_binary_encode(-z) == 0xFF) and np.all(o.gemlite_binary_encode(z) == 0x00)
    one = z.copy()
    one[2, 5] = 1
    b = o.gemlite_binary_encode(one)
    assert b.shape == (2, 16) and b[0, 2] == 0x20 and np.count_nonzero(b) == 1
    assert np.array_equal(o.gemlite_binary_decode(b, 16, 16), one)
    sq = np.zeros((16, 16), dtype=np.uint8)
    sq[15, 0] = 0x80
    codes = o.gemlite_binary_decode(sq, 16, 128)
    assert codes[0, 127] == 1 and np.count_nonzero(codes == 1) == 1
    rng = np.random.default_rng(seed)
    N, K = 32, 256
    codes = gen_codes(rng, N, K, 1)
    b = o.gemlite_binary_encode(codes)
    bits = np.unpackbits(b[:, :, None], axis=2, bitorder="little")         # [K/8, N, 8]
    direct = 2 * bits.transpose(0, 2, 1).reshape(K, N).T.astype(np.int8) - 1
    assert np.array_equal(direct, codes)
    got = o.gemlite_binary_decode(b, N, K)
    assert np.array_equal(got, codes)
    w, bad = o.pack(got, 1)
    assert bad == 0
    # word j of row n is bytes 4j .. 4j+3 of column n, little-endian
    assert np.array_equal(w, np.ascontiguousarray(b.T).view("<u4"))


IMPORT_PINS = [pin_import_golden, pin_import_other_routes, pin_import_layouts_agree, pin_import_binary]


# ----------------------------------------------------------------------------------------
# 4-bit codes (two's complement nibbles, 8 per word, least significant first)

def pin_int4_hex_words(o, seed=51):
    """4-bit words equal integers parsed from hex strings written most-significant nibble first
    (the digit of c is "0123456789ABCDEF"[c mod 16], looked up, not computed by the packer's
    rule), and unpacking returns every one of the 16 codes."""
    digits = "0123456789ABCDEF"
    rng = np.random.default_rng(seed)
    codes = gen_codes(rng, 6, 64, 4)
    codes[0, :16] = np.arange(-8, 8)
    w, bad = o.pack(codes, 4)
    assert bad == 0 and w.shape == (6, 8)
    for n in range(6):
        for j in range(8):
            chunk = codes[n, 8 * j:8 * j + 8]
            expect = int("".join(digits[int(c) + 16 if c < 0 else int(c)] for c in reversed(chunk)), 16)
            assert int(w[n, j]) == expect, (n, j)
    assert np.array_equal(o.unpack(w, 64, 4), codes)
    # outside [-8, 7]: packed as 0 and counted
    w, bad = o.pack(np.array([[8, -9, 100, 1, 0, 0, 0, 0]], dtype=np.int8), 4)
    assert bad == 3 and int(w[0, 0]) == 0x00001000


def pin_int4_one_hot(o):
    """One nonzero 4-bit code c at (n0, k0): Y[:, n0] = c * S[n0, grp] * X[:, k0] exactly (an
    exact fp64 product), every other column 0; the extreme codes -8 and 7 included."""
    rng = rng_for(7, 98, 0)
    M, N, K, g = 3, 16, 128, 64
    x = gen_x(rng, M, K)
    s = gen_scales(rng, N, K, g)
    xf = o.bf16_bits_to_f64(x)
    for (n0, k0, grp, c0) in ((0, 0, 0, -8), (15, 127, 1, 7), (5, 64, 1, -1), (9, 63, 0, 3)):
        c = np.zeros((N, K), dtype=np.int8)
        c[n0, k0] = c0
        w, _ = o.pack(c, 4)
        y = o.gemm_ref_f64(x, o.unpack(w, K, 4), s, g)
        assert np.array_equal(y[:, n0], c0 * float(s[n0, grp]) * xf[:, k0]), (n0, k0)
        assert not np.any(np.delete(y, n0, axis=1))


def pin_int4_fsum(o):
    """The 4-bit GEMM against math.fsum of exact products (codes up to magnitude 8)."""
    pin_fsum(o, M=16, N=48, K=256, g=64, bits=4, seed=9)


INT4_PINS = [pin_int4_hex_words, pin_int4_one_hot, pin_int4_fsum]


# ----------------------------------------------------------------------------------------
# Affine 4-bit groups: w = s * q + b, unsigned levels q in [0, 15] (reading R10)

GOLDEN_U4 = os.path.join(os.path.dirname(__file__), "golden", "pack_u4_words.txt")


def load_golden_u4():
    rows = []
    with open(GOLDEN_U4) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            name, levels, word = [s.strip() for s in line.split("|")]
            rows.append((name, np.array([int(v) for v in levels.split(",")], dtype=np.int64), int(word, 16)))
    return rows


def _affine_case(seed, M, N, K, g):
    rng = rng_for(seed, 97, 0)
    x = gen_x(rng, M, K)
    q = rng.integers(0, 16, size=(N, K))
    s = gen_scales(rng, N, K, g)
    b = (-rng.uniform(0.0, 0.4, size=(N, K // g))).astype(np.float16)
    return x, q, s, b


def pin_u4_words(o, seed=61):
    """Unsigned level words equal the hand-worked golden words and integers parsed from hex
    strings written most-significant nibble first (the digit of q looked up in
    "0123456789ABCDEF", not computed by the packer's rule); unpacking returns the levels;
    levels outside 0 .. 15 are packed as 0 and counted."""
    for name, levels, word in load_golden_u4():
        w, bad = o.pack_u4(levels[None, :])
        assert bad == 0 and w.shape == (1, 1) and int(w[0, 0]) == word, f"{name}: {int(w[0, 0]):#010x}"
        assert np.array_equal(o.unpack_u4(np.array([[word]], dtype=np.uint32), 8)[0], levels), name
    digits = "0123456789ABCDEF"
    q = np.random.default_rng(seed).integers(0, 16, size=(5, 64))
    w, bad = o.pack_u4(q)
    assert bad == 0 and w.shape == (5, 8)
    for n in range(5):
        for j in range(8):
            assert int(w[n, j]) == int("".join(digits[int(v)] for v in reversed(q[n, 8 * j:8 * j + 8])), 16), (n, j)
    assert np.array_equal(o.unpack_u4(w, 64), q)
    w, bad = o.pack_u4(np.array([[16, -1, 200, 1, 0, 0, 15, 0]]))
    assert bad == 3 and int(w[0, 0]) == 0x0F001000


def pin_affine_group_sums(o):
    """X = 1 on the run of group j of row j (0 elsewhere): Y[j, n] = s[n, j] * (sum of the run's
    levels) + g * b[n, j], a closed form evaluated with integer level sums.  A bias taken from
    the wrong group, dropped, or multiplied by the level fails it."""
    g, G = 64, 4
    K, N = g * G, 16
    _, q, s, b = _affine_case(5, 1, N, K, g)
    x = np.zeros((G, K), dtype=np.uint16)
    for j in range(G):
        x[j, j * g:(j + 1) * g] = 0x3F80  # bf16 1.0
    w, _ = o.pack_u4(q)
    y = o.gemm_affine_ref_f64(x, o.unpack_u4(w, K), s, b, g)
    for j in range(G):
        for n in range(N):
            want = float(s[n, j]) * int(q[n, j * g:(j + 1) * g].sum()) + g * float(b[n, j])
            assert abs(y[j, n] - want) <= 1e-12 * (abs(want) + 1), (j, n, y[j, n], want)


def pin_affine_is_symmetric_shifted(o, seed=63):
    """With b = -8 s (exact in fp16) and q = c + 8 for two's complement codes c in [-8, 7], the
    affine weight equals the symmetric 4-bit weight s * c: the affine GEMM must equal the pinned
    symmetric oracle exactly, through packing and unpacking of the levels."""
    M, N, K, g = 8, 32, 256, 64
    x, _, s, _ = _affine_case(seed, M, N, K, g)
    c = gen_codes(rng_for(seed, 97, 1), N, K, 4)
    b = (np.float16(-8.0) * s).astype(np.float16)
    assert np.array_equal(b.astype(np.float64), -8.0 * s.astype(np.float64))
    w, bad = o.pack_u4(c.astype(np.int64) + 8)
    assert bad == 0
    y = o.gemm_affine_ref_f64(x, o.unpack_u4(w, K), s, b, g)
    assert np.array_equal(y, o.gemm_ref_f64(x, c, s, g))


def pin_affine_fsum(o, seed=65):
    """The affine GEMM against math.fsum of its exact terms, within the fp64 summation bound."""
    M, N, K, g = 6, 24, 256, 64
    x, q, s, b = _affine_case(seed, M, N, K, g)
    y = o.gemm_affine_ref_f64(x, q, s, b, g)
    xf = o.bf16_bits_to_f64(x)
    wabs = np.abs(q * np.repeat(s.astype(np.float64), g, 1)) + np.abs(np.repeat(b.astype(np.float64), g, 1))
    bound = 4 * K * 2.0 ** -53 * (np.abs(xf) @ wabs.T)
    for m in range(M):
        for n in range(N):
            e = o.gemm_affine_fsum_element(x, q, s, b, g, m, n)
            assert abs(y[m, n] - e) <= bound[m, n] + 1e-300, (m, n)


def pin_affine_bias_only(o, seed=67):
    """Zero scales leave only the bias term: Y[m, n] = sum_g b[n, g] * (sum of X[m, k] over group
    g), evaluated with math.fsum over the activations of each group (no weight is formed)."""
    M, N, K, g = 4, 16, 192, 64
    x, q, s, b = _affine_case(seed, M, N, K, g)
    s = np.zeros_like(s)
    y = o.gemm_affine_ref_f64(x, q, s, b, g)
    xf = o.bf16_bits_to_f64(x)
    for m in range(M):
        rs = [math.fsum(float(v) for v in xf[m, j * g:(j + 1) * g]) for j in range(K // g)]
        for n in range(N):
            want = math.fsum(float(b[n, j]) * rs[j] for j in range(K // g))
            assert abs(y[m, n] - want) <= 1e-12 * (abs(want) + 1), (m, n)


AFFINE_PINS = [pin_u4_words, pin_affine_group_sums, pin_affine_is_symmetric_shifted, pin_affine_fsum,
               pin_affine_bias_only]
