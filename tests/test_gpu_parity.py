"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Indices: bit-exact except near-ties (oracle gap < 1e-5), which are counted and
checked for validity.  Weights: within 1e-5.  Outputs relative to the output
RMS: bf16 max 2e-2 / mean 2e-3; fp32 max 1e-5.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import workloads as wl
from workloads.device import stream_layer, to_device, upload_layer
from expert_feed import ExpertFeed

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_transformer_glm_amd as glm
else:  # collected on a CPU-only machine: every test here is skipped
    glm = None


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def run_layer(dev, k=None, scale=None, workspace=None):
    w = dev.w
    k = w.k if k is None else k
    scale = w.scale if scale is None else scale
    T = dev.x.shape[0]
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    wt = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, dev.x.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    glm.forward(*dev.args(), k, scale, out=out, topk_idx=idx, topk_w=wt, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


def check(L, out, idx, wt, k=None, scale=None, sample=None, label="", ref=None):
    w = L.w
    k = w.k if k is None else k
    scale = w.scale if scale is None else scale
    rep = parity.compare_routing(idx, wt, L.x, L.router_w, L.corr_bias, k, scale, ref=ref)
    assert rep.ok, f"{label}: invalid routing on tokens {rep.invalid[:10]}"
    assert rep.max_weight_err <= parity.WEIGHT_TOL, f"{label}: weight err {rep.max_weight_err}"
    toks = np.arange(out.shape[0]) if sample is None else np.asarray(sample)
    get = lambda e: (L.w1[e], L.w3[e], L.w2[e])
    feed = ExpertFeed(get, np.unique(rep.forced_idx[toks])) if L.w.E * L.w.F * L.w.D > 1 << 30 \
        else get
    try:
        ref, _ = oracle.forward(L.x[toks], L.router_w, L.corr_bias, feed, (L.sw1, L.sw3, L.sw2),
                                k, scale, force_idx=rep.forced_idx[toks])
    finally:
        if feed is not get:
            feed.close()
    o = parity.compare_output(out[toks], ref)
    log(f"{label}: tokens={rep.tokens} exact={rep.exact} near-tie={rep.excused} "
        f"max|dw|={rep.max_weight_err:.2e} out max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e} "
        f"(compared {len(toks)} tokens)")
    if w.dtype == "f32":
        assert o.max_rel <= parity.F32_MAX_REL, label
    else:
        assert o.max_rel <= parity.BF16_MAX_REL, label
        assert o.mean_rel <= parity.BF16_MEAN_REL, label
    return rep, o


def W(base="mid_bf16", **kw):
    return wl.WORKLOADS[base].with_(**kw)


SMALL = {
    "tiny_f32": wl.WORKLOADS["tiny_f32"],
    "mid_bf16": wl.WORKLOADS["mid_bf16"],
    "ragged_fs192": W(name="ragged_fs192", T=37, D=256, E=16, k=3, F=128, Fs=192, seed=11,
                      weight_seed=11),
    "single_token": W(name="single_token", T=1, D=64, E=4, k=1, F=64, Fs=64, seed=12,
                      weight_seed=12),
    "e40_k6": W(name="e40_k6", T=200, D=192, E=40, k=6, F=64, Fs=128, seed=13, weight_seed=13),
    "k_equals_e": W(name="k_equals_e", T=70, D=128, E=8, k=8, F=64, Fs=64, seed=14,
                    weight_seed=14),
    "e256_k8_small": W(name="e256_k8_small", T=130, D=128, E=256, k=8, F=64, Fs=64, seed=15,
                       weight_seed=15),
    "many_tokens": W(name="many_tokens", T=5000, D=256, E=64, k=4, F=128, Fs=128, seed=16,
                     weight_seed=16),
    "mid_rows": W(name="mid_rows", T=600, D=256, E=32, k=2, F=128, Fs=64, seed=17,
                  weight_seed=17),
    "top32": W(name="top32", T=50, D=128, E=64, k=32, F=64, Fs=64, seed=18, weight_seed=18),
    # ~160 rows per expert: 256-row tiles with the copy-before-wait hand-over
    # in both grouped GEMMs (gate/up K = 256, down K = 256: four K steps each,
    # so both run the refill-then-wait order and its tail), every output
    # element compared
    "early_rows": W(name="early_rows", T=640, D=256, E=8, k=2, F=256, Fs=256, seed=21,
                    weight_seed=21),
    # >160 rows per expert on 256-row tiles (split rings): gate/up K = 512 and
    # down K = 384 (8 and 6 K steps: every position of the six-step ring
    # period, prologue and tail); an odd gate/up K step count (7) with D = 448
    "big_even": W(name="big_even", T=3000, D=512, E=16, k=2, F=384, Fs=384, seed=23,
                  weight_seed=23),
    "big_odd": W(name="big_odd", T=2600, D=448, E=16, k=2, F=256, Fs=256, seed=24,
                 weight_seed=24),
    # 768-wide K (12 steps): the steady six-step loop runs once before the tail
    "big_k768": W(name="big_k768", T=2400, D=768, E=12, k=2, F=256, Fs=256, seed=25,
                  weight_seed=25),
    "f32_ragged": W("tiny_f32", name="f32_ragged", T=37, D=100, E=5, k=2, F=30, Fs=7, seed=19,
                    weight_seed=19),
    "f32_many": W("tiny_f32", name="f32_many", T=300, D=64, E=16, k=4, F=32, Fs=48, seed=20,
                  weight_seed=20),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(name):
    w = SMALL[name]
    L = wl.make_layer(w, threads=4)
    out, idx, wt = run_layer(upload_layer(L))
    check(L, out, idx, wt, label=name)


def test_route_entry_matches_forward_routing():
    L = wl.make_layer(wl.WORKLOADS["mid_bf16"], threads=4)
    dev = upload_layer(L)
    _, idx_f, w_f = run_layer(dev)
    idx, wt = glm.route(dev.x, dev.router_w, dev.corr_bias, L.w.k, L.w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_f)
    np.testing.assert_array_equal(wt.cpu().numpy(), w_f)
    rep = parity.compare_routing(idx.cpu().numpy(), wt.cpu().numpy(), L.x, L.router_w,
                                 L.corr_bias, L.w.k, L.w.scale)
    assert rep.ok and rep.max_weight_err <= parity.WEIGHT_TOL
    assert rep.weight_sum_err <= 2e-6


def test_plain_entry_points_through_ctypes():
    """glm_moe_route and glm_moe_forward themselves (no options, no trace),
    with the workspace sized by glm_moe_workspace_bytes, against the oracle."""
    import ctypes
    from sparse_moe_transformer_glm_amd._lib import Dims

    w = wl.WORKLOADS["mid_bf16"]
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    lib = glm.lib()
    d = Dims(w.T, w.D, w.E, w.F, w.Fs, glm.BF16, glm.BF16)
    n = lib.glm_moe_workspace_bytes(ctypes.byref(d), w.k)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    x, rw, cb, w1, w3, w2, sw1, sw3, sw2 = (t.data_ptr() for t in dev.args())

    def fresh():
        return (torch.full((w.T, w.k), -1, dtype=torch.int32, device="cuda"),
                torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda"),
                torch.full((w.T, w.D), float("nan"), dtype=torch.float32, device="cuda"))

    ridx, rwt, _ = fresh()
    st = lib.glm_moe_route(ctypes.byref(d), x, rw, cb, w.k, w.scale, ridx.data_ptr(),
                           rwt.data_ptr(), ws.data_ptr(), n, s)
    assert st == glm.OK, lib.glm_moe_last_error()
    idx, wt, out = fresh()
    st = lib.glm_moe_forward(ctypes.byref(d), x, rw, cb, w1, w3, w2, sw1, sw3, sw2, w.k, w.scale,
                             out.data_ptr(), idx.data_ptr(), wt.data_ptr(), ws.data_ptr(), n, s)
    assert st == glm.OK, lib.glm_moe_last_error()
    _, _, out_noroute = fresh()  # routing outputs are nullable
    st = lib.glm_moe_forward(ctypes.byref(d), x, rw, cb, w1, w3, w2, sw1, sw3, sw2, w.k, w.scale,
                             out_noroute.data_ptr(), None, None, ws.data_ptr(), n, s)
    assert st == glm.OK, lib.glm_moe_last_error()
    torch.cuda.synchronize()
    out, idx, wt = out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()
    np.testing.assert_array_equal(ridx.cpu().numpy(), idx)
    np.testing.assert_array_equal(rwt.cpu().numpy(), wt)
    np.testing.assert_array_equal(out_noroute.cpu().numpy(), out)
    check(L, out, idx, wt, label="plain entry points")


def test_weights_sum_to_scale_and_k1_exact():
    L = wl.make_layer(wl.WORKLOADS["mid_bf16"], threads=4)
    dev = upload_layer(L)
    _, _, wt = run_layer(dev)
    assert np.abs(wt.sum(1) - 2.5).max() <= 2e-6
    _, idx1, wt1 = run_layer(dev, k=1)
    assert (wt1 == 2.5).all()


def test_deterministic_bitwise():
    L = wl.make_layer(wl.WORKLOADS["mid_bf16"], threads=4)
    dev = upload_layer(L)
    a = run_layer(dev)
    b = run_layer(dev)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_exact_ties_go_to_lower_index():
    w = W(name="ties", T=256, D=128, E=16, k=4, F=64, Fs=64, seed=21, weight_seed=21)
    L = wl.make_layer(w, threads=4)
    L.router_w[9] = L.router_w[3]
    L.corr_bias[9] = L.corr_bias[3] = np.float32(0.3)
    L.router_w[12] = L.router_w[5]
    L.corr_bias[12] = L.corr_bias[5] = np.float32(10.0)  # always selected, first two slots
    out, idx, wt = run_layer(upload_layer(L))
    assert (idx[:, 0] == 5).all() and (idx[:, 1] == 12).all()
    for t in range(w.T):
        row = idx[t].tolist()
        if 9 in row:
            assert 3 in row and row.index(3) < row.index(9), (t, row)
    check(L, out, idx, wt, label="ties")


def test_scale_zero_is_shared_only():
    L = wl.make_layer(wl.WORKLOADS["mid_bf16"], threads=4)
    dev = upload_layer(L)
    out0, idx0, wt0 = run_layer(dev, scale=0.0)
    assert (wt0 == 0).all()
    check(L, out0, idx0, wt0, scale=0.0, label="scale0")
    dev.w2.zero_()
    outz, _, _ = run_layer(dev)
    np.testing.assert_array_equal(out0, outz)


def test_identity_experts_closed_form():
    T, D, E, F, k = 64, 128, 8, 64, 2
    w = W(name="identity", T=T, D=D, E=E, k=k, F=F, Fs=F, seed=22, weight_seed=22)
    L = wl.make_layer(w, threads=4)
    perm = np.random.default_rng(5).permutation(D)[:F]
    one, two = np.uint16(0x3F80), np.uint16(0x4000)
    L.w1[:] = 0
    L.w3[:] = 0
    L.w2[:] = 0
    L.sw1[:] = 0
    L.sw3[:] = 0
    L.sw2[:] = 0
    for f in range(F):
        L.w1[:, f, f] = one
        L.w3[:, f, f] = two
        L.sw1[f, f] = one
        L.sw3[f, f] = two
        L.sw2[perm[f], f] = one
        for e in range(E):
            L.w2[e, perm[f], f] = wl.f32_to_bf16_bits(np.array([e + 1.0], np.float32))[0]
    out, idx, wt = run_layer(upload_layer(L))
    x = oracle.decode(L.x)
    want = np.zeros((T, D))
    for t in range(T):
        coef = sum(wt[t, j] * (idx[t, j] + 1.0) for j in range(k)) + 1.0
        g = x[t, :F]
        want[t, perm] = coef * (g / (1.0 + np.exp(-g))) * (2.0 * g)
    # Every weight here is exact in bf16, so the only lossy step is the bf16
    # rounding of the gated hidden value (relative 2^-9); each output element
    # is one such value times fp32 factors.
    err = np.abs(out - want)
    assert (err <= 2.0 ** -8 * np.abs(want) + 1e-6).all(), err.max()
    rows = np.setdiff1d(np.arange(D), perm)
    assert (out[:, rows] == 0).all()
    rep = parity.compare_routing(idx, wt, L.x, L.router_w, L.corr_bias, k, w.scale)
    assert rep.ok and rep.max_weight_err <= parity.WEIGHT_TOL


def test_zero_tokens_leaves_output_untouched():
    w = wl.WORKLOADS["mid_bf16"]
    L = wl.make_layer(w.with_(T=4), threads=4)
    dev = upload_layer(L)
    dev.x = dev.x[:0]
    out = torch.full((0, w.D), 1.0, device="cuda")
    glm.forward(*dev.args(), w.k, w.scale, out=out)
    torch.cuda.synchronize()


def test_workspace_reuse_across_sizes():
    """One workspace sized for the larger call serves a smaller one after it."""
    w = wl.WORKLOADS["mid_bf16"]
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    ws = glm.new_workspace(w.T, w.D, w.E, w.F, w.Fs, w.k, torch.bfloat16)
    big = run_layer(dev, workspace=ws)
    dev_small = upload_layer(L)
    dev_small.x = dev.x[:100].contiguous()
    small = run_layer(dev_small, workspace=ws)
    np.testing.assert_array_equal(small[1], big[1][:100])
    np.testing.assert_array_equal(small[2], big[2][:100])
    # tokens are independent, but tile boundaries differ: compare to tolerance
    o = parity.compare_output(small[0], big[0][:100])
    assert o.max_rel <= 1e-6


def test_error_codes_raise():
    w = wl.WORKLOADS["mid_bf16"]
    L = wl.make_layer(w.with_(T=8), threads=4)
    dev = upload_layer(L)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(glm.GlmMoeError) as ei:
        glm.forward(*dev.args(), w.k, w.scale, workspace=ws)
    assert ei.value.status == glm.EWORKSPACE
    with pytest.raises(glm.GlmMoeError) as ei:
        glm.forward(*dev.args(), 40, w.scale)
    assert ei.value.status == glm.EINVAL


# ------------------------------------------------------------ GLM shape

@pytest.fixture(scope="module")
def glm_layer():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    t0 = time.time()
    w = wl.WORKLOADS["glm_prefill"]
    log("drawing and uploading the GLM-5.2-shape layer (256 experts, 19.3 GB bf16)")
    dev, host = stream_layer(w, keep_host=True)
    log(f"layer ready in {time.time() - t0:.1f}s")
    return dev, host


def _glm_case(glm_layer, name):
    dev, host = glm_layer
    w = wl.WORKLOADS[name]
    assert (w.D, w.E, w.F, w.Fs, w.weight_seed) == (host.w.D, host.w.E, host.w.F, host.w.Fs,
                                                    host.w.weight_seed)
    L = wl.HostLayer(w, wl.make_x(w), host.router_w, wl.make_corr_bias(w), host.w1, host.w3,
                     host.w2, host.sw1, host.sw3, host.sw2)
    d = type(dev)(w, to_device(L.x), dev.router_w, to_device(L.corr_bias), dev.w1, dev.w3,
                  dev.w2, dev.sw1, dev.sw3, dev.sw2)
    return L, d


def _sample(T, n, extra=()):
    rng = np.random.default_rng(2024)
    picks = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    picks |= {0, T - 1} | {t for t in (63, 64, 127, 128, T // 2) if t < T}
    picks |= set(int(t) for t in extra)
    return np.array(sorted(picks))


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_sample", [("glm_decode", None), ("glm_prefill", 1024),
                                           ("glm_chunk_2k", 1024), ("glm_skew", 1024),
                                           ("glm_skew_mild", 1024)])
def test_glm_shape(glm_layer, name, n_sample):
    L, dev = _glm_case(glm_layer, name)
    t0 = time.time()
    out, idx, wt = run_layer(dev)
    log(f"{name}: GPU layer done ({time.time() - t0:.1f}s incl. readback)")
    load = oracle.expert_load(idx, L.w.E)
    log(f"{name}: experts used {int((load > 0).sum())}/{L.w.E}, rows per expert "
        f"max {load.max()} mean {load.mean():.1f}, hot(0..15) share "
        f"{load[:16].sum() / load.sum():.3f}")
    assert np.isfinite(out).all()
    ref = oracle.route(L.x, L.router_w, L.corr_bias, L.w.k, L.w.scale)
    sample = None
    if n_sample is not None:
        near = np.nonzero((idx != ref.idx).any(1))[0]
        sample = _sample(L.w.T, n_sample, extra=near[:4])
    check(L, out, idx, wt, sample=sample, label=name, ref=ref)
    log(f"{name}: checked in {time.time() - t0:.1f}s")


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_glm_shape_block_with_group_routing(glm_layer):
    """GLM-5.2 shape, decode batch, with the pre-norm block around the layer
    (RMSNorm in, residual add out) and group-limited routing (8 groups of 32,
    4 kept, scale 1.0)."""
    L, dev = _glm_case(glm_layer, "glm_decode")
    w = L.w
    h, nw = wl.make_hidden(w), wl.make_norm_weight(w)
    groups = dict(n_group=8, topk_group=4, group_topk=2)
    eps, scale = 1e-5, 1.0
    T = w.T
    idx = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
    wt = torch.full((T, w.k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, w.D), float("nan"), dtype=torch.float32, device="cuda")
    a = list(dev.args())
    a[0] = to_device(h)
    glm.forward(*a, w.k, scale, out=out, topk_idx=idx, topk_w=wt, norm_weight=to_device(nw),
                norm_eps=eps, residual=True, **groups)
    torch.cuda.synchronize()
    out, idx, wt = out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()
    xn = oracle.round_bf16(oracle.rmsnorm(h, nw, eps))
    rep = parity.compare_routing(idx, wt, xn, L.router_w, L.corr_bias, w.k, scale, **groups)
    assert rep.ok and rep.max_weight_err <= parity.WEIGHT_TOL
    plain = oracle.route(xn, L.router_w, L.corr_bias, w.k, scale)
    assert (plain.idx != rep.forced_idx).any()
    ref, _ = oracle.block_ffn(
        h, nw, eps, "bf16",
        lambda x: oracle.forward(x, L.router_w, L.corr_bias,
                                 lambda e: (L.w1[e], L.w3[e], L.w2[e]), (L.sw1, L.sw3, L.sw2),
                                 w.k, scale, force_idx=rep.forced_idx))
    base = oracle.decode(h)
    o = parity.compare_output(out - base, ref - base)
    log(f"glm block+groups: exact={rep.exact} near-tie={rep.excused} ffn max/rms={o.max_rel:.3e} "
        f"mean/rms={o.mean_rel:.3e}")
    assert o.max_rel <= parity.BF16_MAX_REL and o.mean_rel <= parity.BF16_MEAN_REL
