"""Parity on the GPU of the layer's options and the dense FFN entry, through the
C ABI, against the CPU oracle:

* group-limited routing (n_group / topk_group / group_topk) and scale 1.0;
* the pre-norm block: RMSNorm of the residual stream before the layer and the
  residual add after it;
* the dense SiLU-gated FFN of the leading dense layers.

Tolerances are those of the plain layer (indices exact up to near-ties,
weights 1e-5, outputs relative to the output RMS: bf16 2e-2 max / 2e-3 mean,
fp32 1e-5 max).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import workloads as wl
from workloads.device import to_device, upload_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_transformer_glm_amd as glm
else:
    glm = None


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def W(base="mid_bf16", **kw):
    return wl.WORKLOADS[base].with_(**kw)


def run(dev, x=None, k=None, scale=None, **opts):
    w = dev.w
    k = w.k if k is None else k
    scale = w.scale if scale is None else scale
    x = dev.x if x is None else x
    T = x.shape[0]
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    wt = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, x.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    a = list(dev.args())
    a[0] = x
    glm.forward(*a, k, scale, out=out, topk_idx=idx, topk_w=wt, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


def experts(L):
    return lambda e: (L.w1[e], L.w3[e], L.w2[e])


def assert_close(o, dtype, label):
    if dtype == "f32":
        assert o.max_rel <= parity.F32_MAX_REL, (label, o)
    else:
        assert o.max_rel <= parity.BF16_MAX_REL, (label, o)
        assert o.mean_rel <= parity.BF16_MEAN_REL, (label, o)


def check_moe(L, x_in, out, idx, wt, k, scale, groups=None, label="", base=None):
    """Routing of ``x_in`` (the layer's actual input) and output, optionally
    plus ``base`` (the residual stream added by the block)."""
    groups = groups or {}
    rep = parity.compare_routing(idx, wt, x_in, L.router_w, L.corr_bias, k, scale, **groups)
    assert rep.ok, f"{label}: invalid routing on tokens {rep.invalid[:10]}"
    assert rep.max_weight_err <= parity.WEIGHT_TOL, (label, rep.max_weight_err)
    ref, _ = oracle.forward(x_in, L.router_w, L.corr_bias, experts(L), (L.sw1, L.sw3, L.sw2),
                            k, scale, force_idx=rep.forced_idx)
    ffn = out if base is None else out - base
    o = parity.compare_output(ffn, ref)
    log(f"{label}: tokens={rep.tokens} exact={rep.exact} near-tie={rep.excused} "
        f"max|dw|={rep.max_weight_err:.2e} ffn max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e}")
    assert_close(o, L.w.dtype, label)
    if base is not None:
        ob = parity.compare_output(out, base + ref)
        assert_close(ob, L.w.dtype, label + " (with residual)")
    return rep


# ------------------------------------------------------------ group routing

GROUP_CASES = {
    # name: (workload, n_group, topk_group, group_topk, scale)
    "mid_g8_tg4": (W(name="mid_g8", seed=31), 8, 4, 2, 1.0),
    "e256_g8_tg4": (W(name="e256_g8", T=130, D=128, E=256, k=8, F=64, Fs=64, seed=32,
                      weight_seed=32), 8, 4, 2, 1.0),
    "e256_g8_tg4_skew": (W(name="e256_g8_skew", T=200, D=128, E=256, k=8, F=64, Fs=64, seed=33,
                           weight_seed=33, bias_std=0.05, hot_count=16, hot_value=0.3),
                         8, 4, 2, 2.5),
    "g16_exact_fill": (W(name="g16_fill", T=150, D=128, E=64, k=8, F=64, Fs=64, seed=34,
                         weight_seed=34), 16, 2, 2, 1.0),    # kept experts == k
    "g4_top1": (W(name="g4_top1", T=100, D=192, E=32, k=4, F=64, Fs=128, seed=35,
                  weight_seed=35), 4, 1, 3, 1.0),              # one group kept, group_topk 3
    "f32_g4": (W("tiny_f32", name="f32_g4", seed=36, weight_seed=36), 4, 2, 2, 1.0),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_group_routing_parity(name):
    w, ng, tg, gk, scale = GROUP_CASES[name]
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    groups = dict(n_group=ng, topk_group=tg, group_topk=gk)
    out, idx, wt = run(dev, scale=scale, **groups)
    rep = check_moe(L, L.x, out, idx, wt, w.k, scale, groups, label=name)
    # the restriction matters on this input: plain top-k would differ somewhere
    plain = oracle.route(L.x, L.router_w, L.corr_bias, w.k, scale)
    assert (plain.idx != rep.forced_idx).any(), name
    gs = w.E // ng
    for t in range(w.T):
        assert len(set((idx[t] // gs).tolist())) <= tg


def test_group_routing_degenerate_cases_equal_plain_routing():
    L = wl.make_layer(W(name="g_degen", seed=37), threads=4)
    dev = upload_layer(L)
    plain = run(dev)
    # every group kept, or one expert per group with all k groups kept: plain top-k
    for opts in (dict(n_group=8, topk_group=8, group_topk=2),
                 dict(n_group=64, topk_group=64, group_topk=1),
                 dict(n_group=1, topk_group=1, group_topk=0)):
        got = run(dev, **opts)
        for a, b in zip(got, plain):
            np.testing.assert_array_equal(a, b, err_msg=str(opts))


def test_group_route_entry_matches_forward():
    L = wl.make_layer(W(name="g_route", seed=38), threads=4)
    dev = upload_layer(L)
    groups = dict(n_group=8, topk_group=3, group_topk=2)
    _, idx_f, w_f = run(dev, scale=1.0, **groups)
    idx, wt = glm.route(dev.x, dev.router_w, dev.corr_bias, L.w.k, 1.0, **groups)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_f)
    np.testing.assert_array_equal(wt.cpu().numpy(), w_f)


def test_scale_one_is_scale_free():
    """Weights at scale 1.0 are the renormalised scores: they sum to one, and
    the routed part of the output is exactly 1/2.5 of the scale-2.5 one."""
    L = wl.make_layer(W(name="scale1", seed=39, dtype="f32", T=64, D=128, E=16, k=4, F=64,
                        Fs=64), threads=4)
    dev = upload_layer(L)
    o1, i1, w1 = run(dev, scale=1.0)
    o25, i25, w25 = run(dev, scale=2.5)
    np.testing.assert_array_equal(i1, i25)
    assert np.abs(w1.sum(1) - 1.0).max() <= 1e-6
    np.testing.assert_allclose(w25, w1 * 2.5, rtol=1e-6, atol=0)
    check_moe(L, L.x, o1, i1, w1, L.w.k, 1.0, label="scale1")


# ------------------------------------------------------------ pre-norm block

def block_inputs(L):
    h = wl.make_hidden(L.w)
    nw = wl.make_norm_weight(L.w)
    return h, nw


def oracle_xn(h, nw, eps, dtype):
    """The layer input of the block as the oracle forms it (held in the
    activation dtype)."""
    xn = oracle.rmsnorm(h, nw, eps)
    return oracle.round_bf16(xn) if dtype == "bf16" else xn.astype(np.float32).astype(np.float64)


BLOCK_CASES = {
    "mid_bf16": W(name="blk_mid", seed=41),
    "ragged_bf16": W(name="blk_ragged", T=37, D=256, E=16, k=3, F=128, Fs=192, seed=42,
                     weight_seed=42),
    "tiny_f32": W("tiny_f32", name="blk_f32", seed=43),
    "ragged_f32": W("tiny_f32", name="blk_f32r", T=37, D=100, E=5, k=2, F=30, Fs=7, seed=44,
                    weight_seed=44),
}


@pytest.mark.parametrize("name", list(BLOCK_CASES))
@pytest.mark.parametrize("residual", [False, True])
def test_norm_block_parity(name, residual):
    w = BLOCK_CASES[name]
    L = wl.make_layer(w, threads=4)
    h, nw = block_inputs(L)
    dev = upload_layer(L)
    eps = 1e-5 if w.dtype == "bf16" else 1e-6
    out, idx, wt = run(dev, x=to_device(h), norm_weight=to_device(nw), norm_eps=eps,
                       residual=residual)
    xn = oracle_xn(h, nw, eps, w.dtype)
    base = oracle.decode(h) if residual else None
    check_moe(L, xn, out, idx, wt, w.k, w.scale, label=f"{name} residual={residual}", base=base)
    if residual:
        # oracle.block_ffn is the block as one function; check it agrees
        rep = parity.compare_routing(idx, wt, xn, L.router_w, L.corr_bias, w.k, w.scale)
        ref, _ = oracle.block_ffn(
            h, nw, eps, w.dtype,
            lambda x: oracle.forward(x, L.router_w, L.corr_bias, experts(L),
                                     (L.sw1, L.sw3, L.sw2), w.k, w.scale,
                                     force_idx=rep.forced_idx))
        assert_close(parity.compare_output(out, ref), w.dtype, name + " block_ffn")


def test_residual_add_is_exact():
    """out(residual) == out(no residual) + h in fp32, bit for bit."""
    for w in (W(name="res_bf16", seed=45), W("tiny_f32", name="res_f32", seed=46)):
        L = wl.make_layer(w, threads=4)
        dev = upload_layer(L)
        h = to_device(wl.make_hidden(w))
        plain, _, _ = run(dev, x=h)
        res, _, _ = run(dev, x=h, residual=True)
        want = torch.from_numpy(plain) + h.float().cpu()
        np.testing.assert_array_equal(res, want.numpy(), err_msg=w.name)


def test_norm_with_unit_weight_and_prenormalised_input():
    """A row already of unit RMS with weight 1 and eps 0 passes through the
    norm unchanged up to one rounding, so the layer routes it like the plain
    layer run on the same row."""
    w = W(name="unitnorm", seed=47, dtype="f32", T=64, D=128, E=16, k=4, F=64, Fs=64)
    L = wl.make_layer(w, threads=4)
    x = oracle.decode(L.x)
    x = (x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))).astype(np.float32)
    dev = upload_layer(L)
    ones = torch.ones(w.D, dtype=torch.float32, device="cuda")
    plain = run(dev, x=to_device(x))
    normed = run(dev, x=to_device(x), norm_weight=ones, norm_eps=0.0)
    np.testing.assert_array_equal(normed[1], plain[1])
    o = parity.compare_output(normed[0], plain[0])
    assert o.max_rel <= 1e-5


def test_norm_route_entry_matches_forward():
    L = wl.make_layer(W(name="norm_route", seed=48), threads=4)
    h, nw = block_inputs(L)
    dev = upload_layer(L)
    hd, nwd = to_device(h), to_device(nw)
    _, idx_f, w_f = run(dev, x=hd, norm_weight=nwd)
    idx, wt = glm.route(hd, dev.router_w, dev.corr_bias, L.w.k, L.w.scale, norm_weight=nwd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_f)
    np.testing.assert_array_equal(wt.cpu().numpy(), w_f)


# ------------------------------------------------------------ dense FFN

DENSE_CASES = {
    # name: (workload, dense width)
    "bf16_wide": (W(name="dense_wide", T=300, D=1024, seed=51, weight_seed=51), 512),
    "bf16_narrow": (W(name="dense_narrow", T=37, D=256, seed=52, weight_seed=52), 192),
    "bf16_one_token": (W(name="dense_one", T=1, D=512, seed=53, weight_seed=53), 256),
    "f32_ragged": (W("tiny_f32", name="dense_f32", T=37, D=100, seed=54, weight_seed=54), 30),
}


def run_dense(w, x, dw, **opts):
    T, D = x.shape
    out = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    glm.dense_ffn(x, *[to_device(a) for a in dw], out=out, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", list(DENSE_CASES))
def test_dense_ffn_parity(name):
    w, F = DENSE_CASES[name]
    dw = wl.make_dense(w, F)
    x = wl.make_x(w)
    out = run_dense(w, to_device(x), dw)
    o = parity.compare_output(out, oracle.dense_ffn(x, *dw))
    log(f"dense {name}: max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e}")
    assert_close(o, w.dtype, name)


@pytest.mark.parametrize("name", ["bf16_wide", "f32_ragged"])
def test_dense_block_parity(name):
    w, F = DENSE_CASES[name]
    dw = wl.make_dense(w, F)
    h, nw = wl.make_hidden(w), wl.make_norm_weight(w)
    out = run_dense(w, to_device(h), dw, norm_weight=to_device(nw), norm_eps=1e-5,
                    residual=True)
    ref, _ = oracle.block_ffn(h, nw, 1e-5, w.dtype, lambda x: (oracle.dense_ffn(x, *dw), None))
    base = oracle.decode(h)
    o = parity.compare_output(out - base, ref - base)
    log(f"dense block {name}: ffn max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e}")
    assert_close(o, w.dtype, name)


def test_dense_zero_tokens():
    w, F = DENSE_CASES["bf16_narrow"]
    dw = [to_device(a) for a in wl.make_dense(w, F)]
    x = torch.empty((0, w.D), dtype=torch.bfloat16, device="cuda")
    out = glm.dense_ffn(x, *dw)
    torch.cuda.synchronize()
    assert out.shape == (0, w.D)


# Dense layers on decode-size batches split their few tiles over K: gate/up
# runs whole tiles until every CU has one and the remaining column tiles in K
# chunks (fixup kernel adds the chunks), or every tile in chunks when there
# are fewer tiles than CUs; down splits every tile.  Each case takes another
# branch of that plan: (T, D, dense width).
DENSE_SPLIT_CASES = {
    "rows32_whole_and_chunks": (16, 6144, 18432),   # 32-row tiles, 256 whole + 32 x 8 chunks
    "rows64_two_row_tiles": (96, 6144, 18432),      # 64-row tiles, 2 row tiles, 512 whole + 64 x 4
    "all_chunks_2": (48, 2048, 2048),               # 32 tiles < CUs: every tile in 2 chunks
    "all_chunks_4": (64, 4096, 1536),               # 24 tiles: every tile in 4 chunks
}


@pytest.mark.parametrize("name", list(DENSE_SPLIT_CASES))
@pytest.mark.timeout(600)
def test_dense_decode_k_split(name):
    T, D, F = DENSE_SPLIT_CASES[name]
    w = wl.WORKLOADS["glm_decode"].with_(name=f"dense_split_{name}", T=T, D=D, seed=61,
                                         weight_seed=61)
    t0 = time.time()
    dw = wl.make_dense(w, F)
    x = wl.make_x(w)
    out = run_dense(w, to_device(x), dw)
    o = parity.compare_output(out, oracle.dense_ffn(x, *dw))
    log(f"dense K split {name} (T={T}, D={D}, F={F}): max/rms={o.max_rel:.3e} "
        f"mean/rms={o.mean_rel:.3e} ({time.time() - t0:.1f}s)")
    assert_close(o, "bf16", f"dense K split {name}")
    again = run_dense(w, to_device(x), dw)
    assert np.array_equal(out, again), "dense K split is not deterministic"


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_dense_glm_width():
    """hidden 6144, dense width 18432, 64 tokens (decode) and a ragged 300."""
    for T in (64, 300):
        w = wl.WORKLOADS["glm_decode"].with_(name=f"dense_glm_{T}", T=T)
        t0 = time.time()
        dw = wl.make_dense(w, wl.GLM_DENSE_WIDTH)
        x = wl.make_x(w)
        out = run_dense(w, to_device(x), dw)
        o = parity.compare_output(out, oracle.dense_ffn(x, *dw))
        log(f"dense GLM width T={T}: max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e} "
            f"({time.time() - t0:.1f}s)")
        assert_close(o, "bf16", f"dense T={T}")
