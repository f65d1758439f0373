"""The seeded input generator: determinism, encoding and distributions (no GPU)."""
import numpy as np

import workloads as wl


def test_streams_are_deterministic_and_independent():
    w = wl.WORKLOADS["mid_bf16"]
    a1, b1, c1 = wl.make_expert(w, 3)
    a2, b2, c2 = wl.make_expert(w, 3)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(c1, c2)
    a4, _, _ = wl.make_expert(w, 4)
    assert not np.array_equal(a1, a4)
    assert not np.array_equal(a1, b1)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.00390625, 1.0078125 + 2 ** -9, 1.01171875, -2.5, 1e-3], np.float32)
    bits = wl.f32_to_bf16_bits(f)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa (1.0)
    assert back[1] == np.float32(1.0)
    # 1 + 2^-7 + 2^-9 rounds to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    # 1 + 3 * 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: goes to even (1 + 2^-6)
    assert back[3] == np.float32(1.015625)
    assert back[4] == np.float32(-2.5)
    assert abs(back[5] - 1e-3) <= 2 ** -9 * 1e-3


def test_distributions():
    w = wl.WORKLOADS["mid_bf16"]
    x = (wl.make_x(w).astype(np.uint32) << 16).view(np.float32)
    assert abs(x.std() - 1.0) < 0.01
    W = wl.make_router_w(w)
    assert abs(W.std() * np.sqrt(w.D) - 1.0) < 0.02
    w1, _, w2 = wl.make_expert(w, 0)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    assert abs(f(w1).std() * np.sqrt(w.D) - 1.0) < 0.02
    assert abs(f(w2).std() * np.sqrt(w.F) - 1.0) < 0.02
    b = wl.make_corr_bias(wl.WORKLOADS["glm_prefill"])
    assert b.shape == (256,) and 0.005 < b.std() < 0.02


def test_skew_bias():
    b = wl.make_corr_bias(wl.WORKLOADS["glm_skew"])
    assert (b[:16] == np.float32(1.5)).all()
    assert abs(b[16:].std() - 0.05) < 0.02


def test_iter_experts_order_and_window():
    w = wl.WORKLOADS["tiny_f32"]
    es = [e for e, _ in wl.iter_experts(w, threads=3)]
    assert es == list(range(w.E))
    L = wl.make_layer(w, threads=2)
    np.testing.assert_array_equal(L.w2[5], wl.make_expert(w, 5)[2])
