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


def test_mxfp8_encoder_agrees_with_the_oracle_format():
    """The generator's MXFP8 encoder (integer rounding of fp32 bit patterns)
    and the oracle's (float64 frexp/round) are separate code for one format."""
    import oracle
    rng = np.random.default_rng(7)
    a = (rng.standard_normal((40, 256)) * np.exp2(rng.integers(-12, 8, (40, 1)))).astype(np.float32)
    a[5, 32:64] = 0
    a[6, :32] = np.float32(448.0) * np.float32(2.0 ** -3)   # block max exactly at a boundary
    c1, s1 = wl.f32_to_mxfp8(a)
    c2, s2 = oracle.mx.quantize(a.astype(np.float64))
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_mxfp8_layer_shapes():
    w = wl.WORKLOADS["mid_mx"].with_(T=8, E=4)
    L = wl.make_layer(w, threads=2)
    assert L.w1.dtype == np.uint8 and L.w1.shape == (4, w.F, w.D)
    assert L.w1s.shape == (4, w.F, w.D // 32) and L.w2s.shape == (4, w.D, w.F // 32)
    assert L.sw2s.shape == (w.D, w.Fs // 32)
    assert L.x.dtype == np.uint16
    (c, s), _, _ = L.expert(1)
    assert c.shape == (w.F, w.D) and s.shape == (w.F, w.D // 32)


def test_kstep_major_marshalling_is_the_documented_permutation():
    """The upload hands MX scales over as [..., K/128, N, 4]: byte j of dword
    (kt, n) is the row-major scale [n][4kt + j]."""
    import torch
    from workloads.device import kstep_major
    rng = np.random.default_rng(7)
    src = rng.integers(0, 256, (3, 5, 16), dtype=np.uint8)
    got = kstep_major(torch.from_numpy(src)).numpy()
    assert got.shape == (3, 4, 5, 4)
    for m in range(3):
        for kt in range(4):
            for n in range(5):
                for j in range(4):
                    assert got[m, kt, n, j] == src[m, n, 4 * kt + j]
