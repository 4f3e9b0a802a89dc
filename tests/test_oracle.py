"""The oracle against its pins, and planted mistakes that the pins must catch (CPU only)."""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from oracle import lowbit_ref as ref
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS + P.SWIGLU_PINS + P.RESIDUAL_PINS + P.IMPORT_PINS + P.INT4_PINS + P.AFFINE_PINS,
                         ids=lambda f: f.__name__)
def test_pin_holds(pin):
    pin(P.real_oracle())


def _swiglu_swapped(x, codes, scales, g):
    n = codes.shape[0] // 2
    y = oracle.gemm_ref_f64(x, codes, scales, g)
    return oracle.silu_f64(y[:, n:]) * y[:, :n]


def _swiglu_sigmoid(x, codes, scales, g):
    n = codes.shape[0] // 2
    y = oracle.gemm_ref_f64(x, codes, scales, g)
    return 1.0 / (1.0 + np.exp(-y[:, :n])) * y[:, n:]


def _silu_sign(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(a))


SWIGLU_PLANTED = {
    "halves_swapped": dict(swiglu_ref_f64=_swiglu_swapped),
    "sigmoid_not_silu": dict(swiglu_ref_f64=_swiglu_sigmoid),
    "silu_sign_flipped": dict(silu_f64=_silu_sign,
                              swiglu_ref_f64=lambda x, c, s, g: _silu_sign(
                                  oracle.gemm_ref_f64(x, c, s, g)[:, :c.shape[0] // 2]) *
                              oracle.gemm_ref_f64(x, c, s, g)[:, c.shape[0] // 2:]),
}


@pytest.mark.parametrize("name", sorted(SWIGLU_PLANTED))
def test_swiglu_planted_mistake_is_caught(name):
    broken = SimpleNamespace(**{**vars(P.real_oracle()), **SWIGLU_PLANTED[name]})
    failures = []
    for pin in P.SWIGLU_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every SwiGLU pin"


def test_statistics_binary():
    P.pin_statistics(P.real_oracle(), bits=1)


def test_fsum_binary_small():
    P.pin_fsum(P.real_oracle(), M=8, N=32, K=128, g=32, bits=1, seed=2)


# ----------------------------------------------------------------------------------------
# Planted mistakes: each broken oracle must fail at least one pin.
# ----------------------------------------------------------------------------------------

def _broken(**overrides):
    o = P.real_oracle()
    d = dict(vars(o))
    d.update(overrides)
    return SimpleNamespace(**d)


def _pack_swapped_signs(codes, bits):
    return ref.pack(-np.asarray(codes), bits) if bits == 2 else ref.pack(codes, bits)


def _pack_msb_first(codes, bits):
    c = np.asarray(codes)
    per = 32 // bits
    N, K = c.shape
    flipped = c.reshape(N, K // per, per)[:, :, ::-1].reshape(N, K)
    return ref.pack(flipped, bits)


def _unpack_msb_first(words, K, bits):
    c = ref.unpack(words, K, bits)
    per = 32 // bits
    N = c.shape[0]
    return c.reshape(N, K // per, per)[:, :, ::-1].reshape(N, K)


def _unpack_11_as_minus(words, K, bits):
    c = ref.unpack(words, K, bits)
    if bits == 2:
        w = np.asarray(words, dtype=np.uint32)
        for i in range(16):
            f = ((w >> np.uint32(2 * i)) & np.uint32(3)) == 3
            c.reshape(w.shape[0], w.shape[1], 16)[:, :, i][f] = -1
    return c


def _gemm_scale_tiled(x, codes, scales, g):
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    N, K = np.asarray(codes).shape
    w = np.asarray(codes, dtype=np.float64) * np.tile(s, (1, g))  # k -> k % (K/g): wrong grouping
    return ref.bf16_bits_to_f64(x) @ w.T


def _gemm_no_scale(x, codes, scales, g):
    return ref.bf16_bits_to_f64(x) @ np.asarray(codes, dtype=np.float64).T


def _gemm_transposed(x, codes, scales, g):
    c = np.asarray(codes)
    if c.shape[0] == c.shape[1]:
        c = c.T
    return ref.gemm_ref_f64(x, c, scales, g)


def _gemm_f32_accumulate(x, codes, scales, g):
    xf = ref.bf16_bits_to_f64(x).astype(np.float32)
    w = ref.dequant_f64(codes, scales, g).astype(np.float32)
    return (xf @ w.T).astype(np.float64)


def _bf16_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _gemm_x_as_fp16(x, codes, scales, g):
    return _bf16_as_fp16(x) @ ref.dequant_f64(codes, scales, g).T


PLANTED = {
    "ternary_signs_swapped": dict(pack=_pack_swapped_signs),
    "msb_first_pack": dict(pack=_pack_msb_first),
    "msb_first_unpack": dict(unpack=_unpack_msb_first),
    "field11_as_minus_one": dict(unpack=_unpack_11_as_minus),
    "scale_group_tiled": dict(gemm_ref_f64=_gemm_scale_tiled),
    "scale_dropped": dict(gemm_ref_f64=_gemm_no_scale),
    "square_transposed": dict(gemm_ref_f64=_gemm_transposed),
    "fp32_accumulate": dict(gemm_ref_f64=_gemm_f32_accumulate),
    "x_read_as_fp16": dict(gemm_ref_f64=_gemm_x_as_fp16, bf16_bits_to_f64=_bf16_as_fp16),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(name):
    broken = _broken(**PLANTED[name])
    failures = []
    for pin in P.ALL_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every pin"


# ----------------------------------------------------------------------------------------
# Number-format helpers and the acceptance check
# ----------------------------------------------------------------------------------------

def test_bf16_widening_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x4000], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 2.0]
    got = oracle.bf16_bits_to_f64(bits)
    assert list(got) == want


def test_bf16_rounding_known_values():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -2.5, 0.0,
                     2.0 ** -133, 1.5 * 2.0 ** -133, 3.5e38])
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x0001, 0x0002, 0x7F80]
    assert [int(b) for b in oracle.f64_to_bf16_bits_rne(vals)] == want


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    ours = oracle.f64_to_bf16_bits_rne(v)
    # torch rounds float32 -> bfloat16 to nearest even; go through float32 only where that
    # first rounding is exact (values with <= 24 significant bits)
    v32 = v.astype(np.float32).astype(np.float64)
    theirs = torch.from_numpy(v32).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits_rne(v32), theirs)
    assert ours.shape == v.shape


def test_tolerance_check():
    rng = np.random.default_rng(2)
    yref = rng.standard_normal((64, 64)) * 2
    yb = oracle.f64_to_bf16_bits_rne(yref)
    r = oracle.check_tolerance(yb, yref)
    assert r["ok"] and r["rel_frob"] < 2.5e-3
    bad = yref.copy()
    bad[3, 4] += 0.011 * (abs(yref[3, 4]) + 1)
    assert not oracle.check_tolerance(bad, yref)["ok"]
    nan = yref.copy()
    nan[0, 0] = math.nan
    assert not oracle.check_tolerance(nan, yref)["ok"]


def test_invalid_codes_counted():
    c = np.array([[0, 1, -1, 2, -2, 5, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0]], dtype=np.int8)
    w, bad = oracle.pack(c, 2)
    assert bad == 3
    assert np.array_equal(oracle.unpack(w, 16, 2)[0], np.where(np.isin(c[0], [-1, 0, 1]), c[0], 0))
    cb = np.ones((1, 32), dtype=np.int8)
    cb[0, 4] = 0
    cb[0, 9] = 3
    wb, badb = oracle.pack(cb, 1)
    assert badb == 2 and int(wb[0, 0]) == 0xFFFFFFFF & ~((1 << 4) | (1 << 9))


def test_roundtrip_large():
    from workloads import gen_codes, rng_for
    for bits in (1, 2):
        c = gen_codes(rng_for(0, 50, bits), 96, 1024, bits)
        w, bad = oracle.pack(c, bits)
        assert bad == 0 and w.shape == (96, 1024 * bits // 32)
        assert np.array_equal(oracle.unpack(w, 1024, bits), c)


def _residual_gate_on_rows(x, c, s, g, r, gt):
    """the gate indexed by output row m instead of feature n (M <= N in the pins)"""
    y = oracle.gemm_ref_f64(x, c, s, g)
    return oracle.bf16_bits_to_f64(r) + oracle.bf16_bits_to_f64(gt)[: y.shape[0], None] * y


def _residual_no_gate(x, c, s, g, r, gt):
    return oracle.bf16_bits_to_f64(r) + oracle.gemm_ref_f64(x, c, s, g)


def _residual_gate_on_sum(x, c, s, g, r, gt):
    gt_f = oracle.bf16_bits_to_f64(gt)[None, :]
    return gt_f * (oracle.bf16_bits_to_f64(r) + oracle.gemm_ref_f64(x, c, s, g))


RESIDUAL_PLANTED = {
    "gate_dropped": dict(residual_ref_f64=_residual_no_gate),
    "gate_on_rows": dict(residual_ref_f64=_residual_gate_on_rows),
    "gate_scales_residual_too": dict(residual_ref_f64=_residual_gate_on_sum),
}


@pytest.mark.parametrize("name", sorted(RESIDUAL_PLANTED))
def test_residual_planted_mistake_is_caught(name):
    broken = SimpleNamespace(**{**vars(P.real_oracle()), **RESIDUAL_PLANTED[name]})
    failures = []
    for pin in P.RESIDUAL_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every residual pin"


# planted importer mistakes: each changes the decoder and its matching encoder alike, so a
# round trip alone would not see it


def _gl_msb_decode(src, N, K, zero=1):
    b = np.asarray(src, dtype=np.uint8)
    q = np.stack([(b[k // 4, :] >> (6 - 2 * (k % 4))) & 3 for k in range(K)], axis=1)
    return ref._level_codes(q, zero)


def _gl_msb_encode(codes, zero=1):
    c = np.asarray(codes, dtype=np.int64) + zero
    out = np.zeros((c.shape[1] // 4, c.shape[0]), dtype=np.uint8)
    for k in range(c.shape[1]):
        out[k // 4, :] |= (c[:, k] << (6 - 2 * (k % 4))).astype(np.uint8)
    return out


def _gl_direct_decode(src, N, K, zero=1):
    b = np.asarray(src, dtype=np.uint8).reshape(N, K // 4)  # the orientation trap
    q = np.stack([(b[:, k // 4] >> (2 * (k % 4))) & 3 for k in range(K)], axis=1)
    return ref._level_codes(q, zero)


def _gl_direct_encode(codes, zero=1):
    c = np.asarray(codes, dtype=np.int64) + zero
    N, K = c.shape
    out = np.zeros((N, K // 4), dtype=np.uint8)
    for k in range(K):
        out[:, k // 4] |= (c[:, k] << (2 * (k % 4))).astype(np.uint8)
    return out.reshape(K // 4, N)


def _mlx_sign_decode(src, N, K, zero=1):
    codes, bad = oracle.mlx_u32_decode(src, N, K, zero)
    return -codes, bad


def _mlx_sign_encode(codes, zero=1):
    return oracle.mlx_u32_encode(-np.asarray(codes, dtype=np.int8), zero)


def _mlx_word_order_decode(src, N, K, zero=1):
    return oracle.mlx_u32_decode(np.asarray(src)[:, ::-1], N, K, zero)


def _mlx_word_order_encode(codes, zero=1):
    return np.ascontiguousarray(oracle.mlx_u32_encode(codes, zero)[:, ::-1])


def _glb_msb_decode(src, N, K):
    b = np.asarray(src, dtype=np.uint8)
    return np.stack([2 * ((b[k // 8, :] >> (7 - k % 8)) & 1).astype(np.int8) - 1 for k in range(K)], axis=1)


def _glb_msb_encode(codes):
    c = np.asarray(codes, dtype=np.int8)
    out = np.zeros((c.shape[1] // 8, c.shape[0]), dtype=np.uint8)
    for k in range(c.shape[1]):
        out[k // 8, :] |= ((c[:, k] == 1).astype(np.uint8) << (7 - k % 8)).astype(np.uint8)
    return out


def _glb_direct_decode(src, N, K):
    b = np.asarray(src, dtype=np.uint8).reshape(N, K // 8)  # the orientation trap
    return np.stack([2 * ((b[:, k // 8] >> (k % 8)) & 1).astype(np.int8) - 1 for k in range(K)], axis=1)


def _glb_direct_encode(codes):
    c = np.asarray(codes, dtype=np.int8)
    N, K = c.shape
    out = np.zeros((N, K // 8), dtype=np.uint8)
    for k in range(K):
        out[:, k // 8] |= ((c[:, k] == 1).astype(np.uint8) << (k % 8)).astype(np.uint8)
    return out.reshape(K // 8, N)


IMPORT_PLANTED = {
    "gemlite_binary_msb_first": dict(gemlite_binary_decode=_glb_msb_decode, gemlite_binary_encode=_glb_msb_encode),
    "gemlite_binary_direct_orientation": dict(gemlite_binary_decode=_glb_direct_decode,
                                              gemlite_binary_encode=_glb_direct_encode),
    "gemlite_msb_first": dict(gemlite_u8t_decode=_gl_msb_decode, gemlite_u8t_encode=_gl_msb_encode),
    "gemlite_direct_orientation": dict(gemlite_u8t_decode=_gl_direct_decode, gemlite_u8t_encode=_gl_direct_encode),
    "mlx_code_sign": dict(mlx_u32_decode=_mlx_sign_decode, mlx_u32_encode=_mlx_sign_encode),
    "mlx_word_order": dict(mlx_u32_decode=_mlx_word_order_decode, mlx_u32_encode=_mlx_word_order_encode),
}


@pytest.mark.parametrize("name", sorted(IMPORT_PLANTED))
def test_import_planted_mistake_is_caught(name):
    broken = SimpleNamespace(**{**vars(P.real_oracle()), **IMPORT_PLANTED[name]})
    failures = []
    for pin in P.IMPORT_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every import pin"


# planted 4-bit mistakes: an unsigned nibble decode, most-significant nibble first (in pack and
# unpack alike), and a scale applied to the wrong group of a 4-bit weight


def _int4_unsigned_unpack(words, K, bits):
    out = oracle.unpack(words, K, bits)
    return (out.astype(np.int64) % 16).astype(np.int8) if bits == 4 else out


def _int4_msb_pack(codes, bits):
    if bits != 4:
        return oracle.pack(codes, bits)
    c = np.asarray(codes, dtype=np.int8)
    w, bad = oracle.pack(c.reshape(c.shape[0], -1, 8)[:, :, ::-1].reshape(c.shape), 4)
    return w, bad


def _int4_msb_unpack(words, K, bits):
    out = oracle.unpack(words, K, bits)
    return out.reshape(out.shape[0], -1, 8)[:, :, ::-1].reshape(out.shape) if bits == 4 else out


INT4_PLANTED = {
    "unsigned_nibbles": dict(unpack=_int4_unsigned_unpack),
    "msb_first_nibbles": dict(pack=_int4_msb_pack, unpack=_int4_msb_unpack),
}


@pytest.mark.parametrize("name", sorted(INT4_PLANTED))
def test_int4_planted_mistake_is_caught(name):
    broken = SimpleNamespace(**{**vars(P.real_oracle()), **INT4_PLANTED[name]})
    failures = []
    for pin in P.INT4_PINS + [P.pin_golden_words]:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every 4-bit pin"


# planted affine 4-bit mistakes: signed nibbles, most-significant nibble first (pack and unpack
# alike), the bias dropped, the bias multiplied by the level, and the first group's bias used for
# every group


def _u4_signed_unpack(words, K):
    q = oracle.unpack_u4(words, K).astype(np.int64)
    return np.where(q >= 8, q - 16, q)


def _u4_msb_pack(levels):
    q = np.asarray(levels)
    return oracle.pack_u4(q.reshape(q.shape[0], -1, 8)[:, :, ::-1].reshape(q.shape))


def _u4_msb_unpack(words, K):
    q = oracle.unpack_u4(words, K)
    return q.reshape(q.shape[0], -1, 8)[:, :, ::-1].reshape(q.shape)


def _affine_with_weight(fn):
    def gemm(x_bits, levels, scales, biases, g):
        q = np.asarray(levels).astype(np.float64)
        s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), g, axis=1)
        b = np.repeat(np.asarray(biases, dtype=np.float16).astype(np.float64), g, axis=1)
        return oracle.bf16_bits_to_f64(x_bits) @ fn(q, s, b, np.asarray(biases, dtype=np.float16), g).T
    return gemm


AFFINE_PLANTED = {
    "u4_signed_nibbles": dict(unpack_u4=_u4_signed_unpack),
    "u4_msb_first": dict(pack_u4=_u4_msb_pack, unpack_u4=_u4_msb_unpack),
    "affine_bias_dropped": dict(gemm_affine_ref_f64=_affine_with_weight(lambda q, s, b, b0, g: q * s)),
    "affine_bias_times_level": dict(gemm_affine_ref_f64=_affine_with_weight(lambda q, s, b, b0, g: q * (s + b))),
    "affine_first_group_bias": dict(gemm_affine_ref_f64=_affine_with_weight(
        lambda q, s, b, b0, g: q * s + b0[:, :1].astype(np.float64))),
}


@pytest.mark.parametrize("name", sorted(AFFINE_PLANTED))
def test_affine_planted_mistake_is_caught(name):
    broken = SimpleNamespace(**{**vars(P.real_oracle()), **AFFINE_PLANTED[name]})
    failures = []
    for pin in P.AFFINE_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passed every affine pin"
