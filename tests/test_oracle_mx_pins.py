"""Pins of the MXFP8 part of the oracle (CPU).

Element decoding and rounding are checked against PyTorch's float8_e4m3fn
type (an independent implementation of the same OCP E4M3 format); the block
exponent against its defining inequality; the MXFP8 layer against a closed
form on identity experts, with the quantisation of the hidden values taken
from PyTorch's rounding.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(v32):
    """E4M3 codes of fp32 values (exact in float64, so one rounding)."""
    t = torch.from_numpy(np.asarray(v32, np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    a, b = mx.decode_e4m3(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    np.testing.assert_array_equal(a[ok], b[ok])
    assert np.isnan(a[0x7F]) and np.isnan(a[0xFF]) and np.isnan(a).sum() == 2


@pytest.mark.parametrize("v,code", [
    (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08),
    (0.0, 0x00), (-0.0, 0x00), (240.0, 0x77), (-1.5, 0xBC),
    (2.0 ** -10, 0x00),          # tie between 0 and 2^-9: even (0)
    (3 * 2.0 ** -10, 0x02),      # tie between 2^-9 and 2^-8: even code 2
    (1.0625, 0x38),              # tie between 1.0 and 1.125: even mantissa (1.0)
    (1.1875, 0x3A),              # tie between 1.125 and 1.25: even mantissa (1.25)
    (1.06251, 0x39),             # just above the tie
    (15.5 * 2.0 ** -9, 0x10),    # tie at the top of a binade: up to 2^-5 (even)
    (15.5 * 2.0 ** -6, 0x28),    # tie at the top of a binade: up to 2^-2 (even)
])
def test_encode_hand_cases(v, code):
    assert int(mx.encode_e4m3(np.array([v]))[0]) == code


def test_encode_matches_torch_on_many_values():
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200000)).astype(np.float32)
    v = (mag * rng.choice([-1, 1], mag.size)).astype(np.float32)
    v = v[np.abs(v) <= 448]
    # include exact midpoints between neighbouring codes
    grid = torch_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    np.testing.assert_array_equal(mx.encode_e4m3(v), torch_encode(v))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        mx.encode_e4m3(np.array([448.5]))


def test_block_exponent_defining_inequality():
    rng = np.random.default_rng(1)
    amax = np.exp2(rng.uniform(-60, 60, 100000))
    amax = np.concatenate([amax, 448.0 * np.exp2(np.arange(-20, 20.0)),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 20.0)), np.inf)])
    s = mx.block_exponent(amax)
    assert np.all(amax <= 448.0 * np.exp2(s.astype(np.float64)))
    assert np.all(amax > 448.0 * np.exp2(s.astype(np.float64) - 1))
    assert list(mx.block_exponent(np.array([448.0, 449.0, 1.0, 0.875, 0.0]))) == [0, 1, -8, -9, 0]


def test_quantize_error_bound_and_no_saturation():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-10, 10, (64, 1)))
    v[3, :32] = 0.0                                 # an all-zero block
    codes, scales = mx.quantize(v)
    assert codes.shape == v.shape and scales.shape == (64, 8)
    assert scales[3, 0] == 127 and np.all(codes[3, :32] == 0)
    s = (scales.astype(np.int64) - 127).repeat(32, axis=1)
    back = mx.dequantize(codes, scales)
    # half a step of E4M3 at the value's binade (2^-10 in units of the scale below 2^-6)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** (s - 10))
    assert np.all(np.abs(back - v) <= bound)
    # the largest element of each block lands in the top binade, none saturates
    top = np.abs(mx.decode_e4m3(codes)).reshape(64, 8, 32).max(axis=-1)
    nz = np.abs(v).reshape(64, 8, 32).max(axis=-1) > 0
    assert np.all(top[nz] > 224 * (1 - 2.0 ** -4)) and np.all(top <= 448)


def test_quantize_is_exact_on_representable_blocks():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, (16, 64)).astype(np.uint8)
    codes[:, ::32] = 0x7A | (codes[:, ::32] & 0x80)  # a magnitude in (224, 448] in every block
    s = rng.integers(-20, 5, (16, 2))
    v = mx.decode_e4m3(codes) * np.exp2(s).repeat(32, axis=1)
    c2, s2 = mx.quantize(v)
    np.testing.assert_array_equal(mx.dequantize(c2, s2), v)
    np.testing.assert_array_equal(s2.astype(np.int64) - 127, s)


def _mx_of_floats(a):
    return mx.quantize(np.asarray(a, np.float64))


def test_forward_mx_identity_experts_closed_form():
    """Identity experts: g = x_f, u = 2 x_f, w2 maps hidden f to output perm[f]
    with factor (e+1); the shared expert the same with factor 1.  The layer must
    give (sum_j w_j (e_j+1) + 1) * Q(SiLU(x_f) * 2 x_f) at perm[f], where x is
    already MXFP8-exact and Q is MXFP8 rounding along the hidden dimension,
    computed here with PyTorch's E4M3 conversion and the block inequality."""
    rng = np.random.default_rng(4)
    T, D, E, F, k = 16, 64, 4, 32, 2
    xc = rng.integers(0, 0x7E, (T, D)).astype(np.uint8)
    xc[:, ::32] = 0x7C                       # 320: block maximum in (224, 448]
    x = mx.decode_e4m3(xc) * 2.0 ** -8
    perm = rng.permutation(D)[:F]
    w1 = np.zeros((F, D)); w3 = np.zeros((F, D))
    w1[np.arange(F), np.arange(F)] = 1.0
    w3[np.arange(F), np.arange(F)] = 2.0
    def w2_of(c):
        w = np.zeros((D, F)); w[perm, np.arange(F)] = c; return w
    experts = {e: (_mx_of_floats(w1), _mx_of_floats(w3), _mx_of_floats(w2_of(e + 1.0)))
               for e in range(E)}
    shared = (_mx_of_floats(w1), _mx_of_floats(w3), _mx_of_floats(w2_of(1.0)))
    W = rng.standard_normal((E, D)) * 0.1
    b = np.zeros(E)
    out, r = oracle.forward_mx(x, W, b, lambda e: experts[e], shared, k, 2.5)
    g = x[:, :F]
    h = g / (1 + np.exp(-g)) * 2 * g
    # Q(h): block exponent from the defining inequality, rounding by PyTorch
    hb = h.reshape(T, F // 32, 32)
    amax = np.abs(hb).max(axis=-1)
    s = np.ceil(np.log2(amax / 448.0))
    s = np.where(amax > 448.0 * np.exp2(s), s + 1, s)
    s = np.where(amax <= 448.0 * np.exp2(s - 1), s - 1, s)
    scaled = hb / np.exp2(s)[..., None]
    # PyTorch rounds through fp32: keep to values whose fp32 rounding cannot
    # move them across an E4M3 midpoint (all of them for this seed)
    grid = torch_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    gap = np.abs(np.abs(scaled)[..., None] - mids).min(axis=-1)
    assert np.all(gap > np.abs(scaled) * 2.0 ** -20)
    q = torch_decode(torch_encode(scaled)) * np.exp2(s)[..., None]
    q = q.reshape(T, F)
    coef = (r.weight * (r.idx + 1.0)).sum(axis=1) + 1.0
    want = np.zeros((T, D))
    want[:, perm] = coef[:, None] * q
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)


def test_forward_mx_w2_scale_is_applied():
    """Raising every w2 block scale by one doubles the routed part exactly."""
    rng = np.random.default_rng(5)
    T, D, E, F, k = 24, 64, 4, 64, 2
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D)) * 0.2
    b = rng.standard_normal(E) * 0.01
    ex = {e: (_mx_of_floats(rng.standard_normal((F, D)) / 8), _mx_of_floats(rng.standard_normal((F, D)) / 8),
              _mx_of_floats(rng.standard_normal((D, F)) / 8)) for e in range(E)}
    zero_shared = (_mx_of_floats(np.zeros((F, D))), _mx_of_floats(np.zeros((F, D))),
                   _mx_of_floats(np.zeros((D, F))))
    out1, _ = oracle.forward_mx(x, W, b, lambda e: ex[e], zero_shared, k, 2.5)
    ex2 = {e: (a, c, (w2[0], (w2[1] + 1).astype(np.uint8))) for e, (a, c, w2) in ex.items()}
    out2, _ = oracle.forward_mx(x, W, b, lambda e: ex2[e], zero_shared, k, 2.5)
    np.testing.assert_array_equal(out2, 2 * out1)
