"""glm_moe_forward_noalloc (the layer in the library's fixed per-GPU buffer)
against glm_moe_forward with a caller workspace, through the C ABI.

Both run the same kernels with the same plan, so routing and output must be
bit-identical.  Two calls in a row, the second with a smaller batch (the
buffer keeps the first call's contents), on a bf16 layer and a 256-expert
top-8 layer; sizes beyond the buffer are rejected before anything runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from workloads.device import upload_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_transformer_glm_amd as glm
    from sparse_moe_transformer_glm_amd._lib import Dims
else:
    glm = None


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _both(dev, T, k, scale):
    args = [dev.x[:T].contiguous()] + list(dev.args()[1:])
    D = args[0].shape[1]
    res = []
    for noalloc in (False, True):
        idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        wt = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            glm.forward_noalloc(*args, k, scale, out, topk_idx=idx, topk_w=wt)
        else:
            glm.forward(*args, k, scale, out=out, topk_idx=idx, topk_w=wt)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()))
    return res


@pytest.mark.parametrize("name,T,T2", [
    ("mid_bf16", 512, 100),
    ("e256_k8", 235, 64),
])
def test_noalloc_matches_forward_two_calls(name, T, T2):
    if name == "mid_bf16":
        w = wl.WORKLOADS["mid_bf16"]
    else:
        w = wl.WORKLOADS["mid_bf16"].with_(name="noalloc_e256", T=T, D=512, E=256, k=8, F=256,
                                           Fs=256, seed=31, weight_seed=31)
    dev = upload_layer(wl.make_layer(w, threads=4))
    for t in (T, T2):  # the second call is smaller and follows the first
        (o_ref, i_ref, w_ref), (o, i, wt) = _both(dev, t, w.k, w.scale)
        np.testing.assert_array_equal(i, i_ref)
        np.testing.assert_array_equal(wt, w_ref)
        np.testing.assert_array_equal(o, o_ref)
        assert np.isfinite(o).all()


def test_noalloc_rejects_sizes_beyond_its_buffer():
    lib = glm.lib()
    T = 236  # GLM-5.2 shape: needs just over 64 MiB of workspace
    d = Dims(T, 6144, 256, 2048, 2048, glm.BF16, glm.BF16)
    assert lib.glm_moe_workspace_bytes(ctypes.byref(d), 8) > 64 << 20
    # the size check precedes any pointer use: nothing is enqueued
    st = lib.glm_moe_forward_noalloc(ctypes.byref(d), None, None, None, None, None, None, None,
                                     None, None, 8, 2.5, None, None, None, None)
    assert st == glm.EWORKSPACE
    assert b"64" in lib.glm_moe_last_error() or b"67108864" in lib.glm_moe_last_error()
