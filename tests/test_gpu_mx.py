"""Parity of the MXFP8-weight layer (glm_moe_forward_mx) with oracle.forward_mx.

Routing as for the bf16 layer (indices exact up to near-ties, weights 1e-5).

The layer quantises its gated hidden values to MXFP8, a rounding decision
taken on the kernel's fp32 value.  A hidden value within the FP8 MFMA's
accumulation error of a rounding midpoint (or a block maximum near a scale
boundary) may round either way, and one E4M3 step is 6-12% of the value, so
no correct kernel matches an oracle that rounds exact values element for
element.  The decisions are therefore taken once, by the kernel, and checked:

* every hidden code and block scale the kernel wrote (read back from the
  workspace) must be the oracle's rounding rule applied to a value within the
  accumulation budget of the oracle's exact value (oracle.parity.
  mx_hidden_check; the budget 2^-13 of the term magnitudes was measured on
  the GPU);
* the layer output must then match the oracle evaluated on those hidden codes
  element by element within the bf16 bounds (max |out - ref| <= 2e-2 and
  mean <= 2e-3 of the output RMS);
* against oracle.forward_mx itself (its own rounding) the mean bound holds too.

On the small cases ``oracle.parity.mx_explain`` also runs as a diagnostic
(logged, not asserted).
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import workloads as wl
from workloads.device import stream_layer, to_device, upload_layer

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


def W(**kw):
    return wl.WORKLOADS["mid_mx"].with_(**kw)


def run(dev, k=None, scale=None, x=None, hidden=False, **opts):
    """One forward_mx call; with ``hidden`` also the gated hidden rows the
    kernels wrote, read back from the workspace in (token, slot) order:
    ((codes [T, k, F], scales [T, k, F/32]), (shared codes [T, Fs], scales))."""
    w = dev.w
    k = w.k if k is None else k
    scale = w.scale if scale is None else scale
    a = list(dev.args())
    if x is not None:
        a[0] = x
    T, D = a[0].shape
    F, Fs = w.F, w.Fs
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    wt = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    o = glm.options(opts.get("n_group", 1), opts.get("topk_group", 1), opts.get("group_topk", 0),
                    opts.get("norm_weight"), opts.get("norm_eps", 1e-5), opts.get("residual", False),
                    D)
    ws = glm.new_workspace(T, D, w.E, F, Fs, k, torch.bfloat16, opts=o, weight=glm.MXFP8)
    glm.forward_mx(*a, k, scale, out=out, topk_idx=idx, topk_w=wt, workspace=ws, **opts)
    torch.cuda.synchronize()
    res = (out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy())
    if not hidden:
        return res
    lay = glm.hidden_layout(T, D, w.E, F, Fs, k, opts=o, weight=glm.MXFP8)
    A = T * k

    def take(off, n):
        return ws[off:off + n].cpu().numpy()

    ra = take(lay.row_assign, 4 * A).view(np.int32)
    hc = take(lay.hidden, A * F).reshape(A, F)
    hs = take(lay.hidden_scale, A * F // 32).reshape(F // 128, A, 4).transpose(1, 0, 2)
    codes = np.empty((A, F), np.uint8)
    scales = np.empty((A, F // 32), np.uint8)
    codes[ra] = hc
    scales[ra] = hs.reshape(A, F // 32)
    sc = take(lay.shared_hidden, T * Fs).reshape(T, Fs)
    ss = take(lay.shared_hidden_scale, T * Fs // 32).reshape(Fs // 128, T, 4).transpose(1, 0, 2)
    return res + (((codes.reshape(T, k, F), scales.reshape(T, k, F // 32)),
                   (sc, ss.reshape(T, Fs // 32))),)


def check(L, x_in, res, k, scale, groups=None, sample=None, label="", base=None, ref=None,
          explain=True):
    out, idx, wt, ((codes, scales), (scodes, sscales)) = res
    groups = groups or {}
    rep = parity.compare_routing(idx, wt, x_in, L.router_w, L.corr_bias, k, scale, ref=ref,
                                 **groups)
    assert rep.ok, f"{label}: invalid routing on tokens {rep.invalid[:10]}"
    assert rep.max_weight_err <= parity.WEIGHT_TOL, (label, rep.max_weight_err)
    toks = np.arange(out.shape[0]) if sample is None else np.asarray(sample)
    want, r = oracle.forward_mx(x_in[toks], L.router_w, L.corr_bias, L.expert, L.shared(), k,
                                scale, force_idx=rep.forced_idx[toks])
    got = out[toks] if base is None else out[toks] - base[toks]
    # the kernel's hidden decisions, each checked against the oracle's value
    xq = oracle.mx.fake_quantize(oracle.decode(x_in[toks]))
    hsum = parity.MxHiddenReport(0, 0, 0, 0, 0, 0, 0)
    def acc(rep_h):
        for f in dataclasses.fields(rep_h):
            setattr(hsum, f.name, getattr(hsum, f.name) + getattr(rep_h, f.name))
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        w1, w3, _ = L.expert(int(e))
        h, eh = parity.mx_hidden_budget(xq[t], w1, w3)
        acc(parity.mx_hidden_check(codes[toks[t], j], scales[toks[t], j], h, eh))
    sw1, sw3, _ = L.shared()
    h, eh = parity.mx_hidden_budget(xq, sw1, sw3)
    acc(parity.mx_hidden_check(scodes[toks], sscales[toks], h, eh))
    on_hidden = oracle.forward_mx_on_hidden(
        r, oracle.mx.dequantize(codes[toks], scales[toks]),
        oracle.mx.dequantize(scodes[toks], sscales[toks]), L.expert, L.shared())
    o = parity.compare_output(got, on_hidden)
    o_plain = parity.compare_output(got, want)
    log(f"{label}: tokens={rep.tokens} exact={rep.exact} near-tie={rep.excused} "
        f"max|dw|={rep.max_weight_err:.2e} hidden values={hsum.values} same={hsum.same} "
        f"other valid rounding={hsum.other_valid} invalid={hsum.invalid} "
        f"(scales other={hsum.scale_other} invalid={hsum.scale_invalid}); "
        f"out vs oracle on these codes max/rms={o.max_rel:.3e} mean/rms={o.mean_rel:.3e}; "
        f"vs oracle's own rounding max/rms={o_plain.max_rel:.3e} mean/rms={o_plain.mean_rel:.3e} "
        f"(compared {len(toks)} tokens)")
    if explain:
        # diagnostic only: its budgets were measured on the GPU
        e = parity.mx_explain(got, want, x_in[toks], r, L.expert, L.shared())
        log(f"{label}: mx_explain: rounding candidates={e.candidates} flips={e.flips} "
            f"max resid/rms={e.max_resid_rel:.2e} unexplained outputs={e.violations}")
    assert hsum.invalid == 0 and hsum.scale_invalid == 0, (label, hsum)
    assert o.max_rel <= parity.BF16_MAX_REL, (label, o)
    assert o.mean_rel <= parity.BF16_MEAN_REL, (label, o)
    assert o_plain.mean_rel <= parity.BF16_MEAN_REL, (label, o_plain)
    return rep, o


CASES = {
    "mid_mx": W(),                                                        # Mid tiles
    "ragged": W(name="mx_ragged", T=37, D=256, E=16, k=3, F=128, Fs=256, seed=61,
                weight_seed=61),                                          # Decode tiles
    "one_token_narrow": W(name="mx_one", T=1, D=128, E=4, k=1, F=128, Fs=128, seed=62,
                          weight_seed=62),                                # narrow down tiles
    "e256_k8": W(name="mx_e256", T=130, D=256, E=256, k=8, F=128, Fs=128, seed=63,
                 weight_seed=63),
    "many_tokens": W(name="mx_many", T=3000, D=256, E=16, k=2, F=256, Fs=128, seed=64,
                     weight_seed=64),                                     # Big tiles
    "mid_rows": W(name="mx_midrows", T=600, D=512, E=32, k=2, F=256, Fs=256, seed=65,
                  weight_seed=65),
    "narrow_d384": W(name="mx_d384", T=70, D=384, E=8, k=2, F=256, Fs=128, seed=66,
                     weight_seed=66),                                     # D % 256 != 0
}


@pytest.mark.parametrize("shape", [(3, 70, 12), (130, 4), (2, 2, 256, 192)])
def test_pack_scales_is_the_kstep_major_permutation(shape):
    """glm_moe_mx_pack_scales against the permutation written out in NumPy:
    byte (kt*N + n)*4 + j of each matrix = row-major scale [n][4kt + j]."""
    rng = np.random.default_rng(sum(shape))
    src = rng.integers(0, 256, shape, dtype=np.uint8)
    *lead, N, KS = shape
    want = np.empty((*lead, KS // 4, N, 4), np.uint8)
    for kt in range(KS // 4):
        for j in range(4):
            want[..., kt, :, j] = src[..., :, 4 * kt + j]
    got = glm.pack_mx_scales(torch.from_numpy(src).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("name", list(CASES))
def test_mx_layer_parity(name):
    w = CASES[name]
    L = wl.make_layer(w, threads=4)
    check(L, L.x, run(upload_layer(L), hidden=True), w.k, w.scale, label=name)


def test_mx_deterministic_and_route_matches_bf16_entry():
    w = CASES["mid_mx"]
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    a, b = run(dev), run(dev)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    idx, wt = glm.route(dev.x, dev.router_w, dev.corr_bias, w.k, w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), a[1])
    np.testing.assert_array_equal(wt.cpu().numpy(), a[2])


def test_mx_block_with_group_routing():
    w = W(name="mx_block", seed=67)
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    h, nw = wl.make_hidden(w), wl.make_norm_weight(w)
    groups = dict(n_group=8, topk_group=4, group_topk=2)
    res = run(dev, x=to_device(h), scale=1.0, hidden=True, norm_weight=to_device(nw),
              norm_eps=1e-5, residual=True, **groups)
    xn = oracle.round_bf16(oracle.rmsnorm(h, nw, 1e-5))
    check(L, xn, res, w.k, 1.0, groups=groups, label="mx block+groups", base=oracle.decode(h))


def test_mx_scale_zero_is_shared_only():
    w = W(name="mx_s0", seed=68)
    L = wl.make_layer(w, threads=4)
    dev = upload_layer(L)
    res = run(dev, scale=0.0, hidden=True)
    assert (res[2] == 0).all()
    check(L, L.x, res, w.k, 0.0, label="mx scale0")


@pytest.fixture(scope="module")
def glm_mx_layer():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    t0 = time.time()
    log("drawing and uploading the GLM-5.2-shape MXFP8 layer (256 experts, 9.9 GB)")
    dev, host = stream_layer(wl.WORKLOADS["glm_prefill_mx"], keep_host=True)
    log(f"layer ready in {time.time() - t0:.1f}s")
    return dev, host


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_sample", [("glm_decode_mx", None), ("glm_prefill_mx", 1024)])
def test_mx_glm_shape(glm_mx_layer, name, n_sample):
    dev, host = glm_mx_layer
    w = wl.WORKLOADS[name]
    L = wl.HostLayer(w, wl.make_x(w), host.router_w, wl.make_corr_bias(w), host.w1, host.w3,
                     host.w2, host.sw1, host.sw3, host.sw2, host.w1s, host.w3s, host.w2s,
                     host.sw1s, host.sw3s, host.sw2s)
    d = dev.with_x(to_device(L.x), to_device(L.corr_bias), w)
    t0 = time.time()
    res = run(d, hidden=True)
    out, idx = res[0], res[1]
    log(f"{name}: GPU layer done ({time.time() - t0:.1f}s incl. readback)")
    assert np.isfinite(out).all()
    ref = oracle.route(L.x, L.router_w, L.corr_bias, w.k, w.scale)
    sample = None
    if n_sample is not None:
        rng = np.random.default_rng(2024)
        near = np.nonzero((idx != ref.idx).any(1))[0]
        sample = np.array(sorted(set(rng.choice(w.T, n_sample, replace=False).tolist())
                                 | {0, w.T - 1} | set(near[:4].tolist())))
    check(L, L.x, res, w.k, w.scale, sample=sample, label=name, ref=ref, explain=False)
