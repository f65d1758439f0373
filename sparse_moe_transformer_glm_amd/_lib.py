"""ctypes binding of ``libglm_moe.so`` (the GLM-5.2 MoE layer C ABI).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  There is no
fallback: if the library is not built, or a tensor is not on the GPU, this
module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # must be imported before the library so both share one HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libglm_moe.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, BF16, MXFP8 = 0, 1, 2
STAGES = ("norm", "router_logits", "router_topk", "scan", "scatter", "gate_up", "down",
          "shared_combine")


class GlmMoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("F", ctypes.c_int32), ("F_shared", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32)]


class Options(ctypes.Structure):
    """``glm_moe_options``: group-limited routing and the pre-norm block."""
    _fields_ = [("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("group_topk", ctypes.c_int32), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("add_residual", ctypes.c_int32)]


class HiddenLayout(ctypes.Structure):
    """``glm_moe_hidden_layout``: workspace offsets of the gated hidden rows."""
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "row_assign", "hidden", "hidden_scale", "shared_hidden", "shared_hidden_scale")]


class MxWeights(ctypes.Structure):
    """``glm_moe_mx_weights``: E4M3 code tensors and their E8M0 scales."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale", "shared_w1", "shared_w1_scale",
        "shared_w3", "shared_w3_scale", "shared_w2", "shared_w2_scale")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_moe_transformer_glm_amd.build` (gfx950 HIP library)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        pd, po = ctypes.POINTER(Dims), ctypes.POINTER(Options)
        L.glm_moe_workspace_size.argtypes = [pd, i32, ctypes.POINTER(sz)]
        L.glm_moe_workspace_size_ex.argtypes = [pd, po, i32, ctypes.POINTER(sz)]
        L.glm_moe_hidden_layout_of.argtypes = [pd, po, i32, ctypes.POINTER(HiddenLayout)]
        L.glm_moe_workspace_bytes.argtypes = [pd, i32]
        L.glm_moe_workspace_bytes.restype = sz
        L.glm_moe_route.argtypes = [pd, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.glm_moe_route_ex.argtypes = [pd, po, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.glm_moe_forward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp,
                                      vp, sz, vp]
        L.glm_moe_forward_traced.argtypes = L.glm_moe_forward.argtypes + [vp]
        L.glm_moe_forward_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32,
                                              vp, vp, vp, vp]
        L.glm_moe_forward_ex.argtypes = [pd, po, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp,
                                         vp, vp, vp, sz, vp, vp]
        L.glm_moe_forward_mx.argtypes = [pd, po, vp, vp, vp, ctypes.POINTER(MxWeights), i32, f32,
                                         vp, vp, vp, vp, sz, vp, vp]
        L.glm_moe_dense_workspace_size.argtypes = [pd, po, ctypes.POINTER(sz)]
        L.glm_moe_dense_ffn.argtypes = [pd, po, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.glm_moe_mx_pack_scales.argtypes = [vp, vp, ctypes.c_int64, i32, i32, vp]
        L.glm_moe_trace_create.argtypes = [ctypes.POINTER(vp), i32]
        L.glm_moe_trace_destroy.argtypes = [vp]
        L.glm_moe_trace_reset.argtypes = [vp]
        L.glm_moe_trace_read.argtypes = [vp, ctypes.POINTER(f32), ctypes.POINTER(i32)]
        L.glm_moe_status_string.argtypes = [i32]
        L.glm_moe_status_string.restype = ctypes.c_char_p
        L.glm_moe_last_error.argtypes = []
        L.glm_moe_last_error.restype = ctypes.c_char_p
        L.glm_moe_version.restype = i32
        for name in ("glm_moe_workspace_size", "glm_moe_workspace_size_ex", "glm_moe_route",
                     "glm_moe_route_ex", "glm_moe_forward", "glm_moe_forward_traced",
                     "glm_moe_forward_ex", "glm_moe_forward_mx", "glm_moe_dense_workspace_size", "glm_moe_dense_ffn",
                     "glm_moe_trace_create", "glm_moe_trace_destroy", "glm_moe_trace_reset",
                     "glm_moe_trace_read", "glm_moe_mx_pack_scales", "glm_moe_hidden_layout_of",
                     "glm_moe_forward_noalloc"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != OK:
        L = lib()
        detail = L.glm_moe_last_error().decode() or L.glm_moe_status_string(status).decode()
        raise GlmMoeError(status, where, detail)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def dims(T: int, D: int, E: int, F: int, Fs: int, dtype: torch.dtype,
         weight: Optional[int] = None) -> Dims:
    """Layer sizes; ``weight`` overrides the weight dtype code (MXFP8)."""
    c = _dtype_code(dtype)
    return Dims(T, D, E, F, Fs, c, c if weight is None else weight)


def options(n_group: int = 1, topk_group: int = 1, group_topk: int = 0,
            norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-5,
            residual: bool = False, D: Optional[int] = None) -> Options:
    """Marshal the layer options (``norm_weight`` is a [D] float32 GPU tensor)."""
    nw = 0
    if norm_weight is not None:
        nw = _ptr(norm_weight, "norm_weight", torch.float32, None if D is None else (D,))
    return Options(int(n_group), int(topk_group), int(group_topk), nw or None, float(norm_eps),
                   1 if residual else 0)


def workspace_size(T: int, D: int, E: int, F: int, Fs: int, top_k: int,
                   dtype: torch.dtype = torch.bfloat16, opts: Optional[Options] = None,
                   weight: Optional[int] = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().glm_moe_workspace_size_ex(ctypes.byref(dims(T, D, E, F, Fs, dtype, weight)),
                                           None if opts is None else ctypes.byref(opts), top_k,
                                           ctypes.byref(n)), "glm_moe_workspace_size_ex")
    return n.value


def workspace_bytes(T: int, D: int, E: int, F: int, Fs: int, top_k: int,
                    dtype: torch.dtype = torch.bfloat16) -> int:
    """``glm_moe_workspace_bytes``: workspace of the plain route/forward calls
    (0 for T = 0; raises on dims those calls would reject)."""
    L = lib()
    n = L.glm_moe_workspace_bytes(ctypes.byref(dims(T, D, E, F, Fs, dtype)), top_k)
    if n == 0 and T > 0:
        raise GlmMoeError(EINVAL, "glm_moe_workspace_bytes", L.glm_moe_last_error().decode())
    return int(n)


def hidden_layout(T: int, D: int, E: int, F: int, Fs: int, top_k: int,
                  dtype: torch.dtype = torch.bfloat16, opts: Optional[Options] = None,
                  weight: Optional[int] = None) -> HiddenLayout:
    """Workspace offsets of the gated hidden rows (``glm_moe_hidden_layout_of``)."""
    lay = HiddenLayout()
    _check(lib().glm_moe_hidden_layout_of(ctypes.byref(dims(T, D, E, F, Fs, dtype, weight)),
                                          None if opts is None else ctypes.byref(opts), top_k,
                                          ctypes.byref(lay)), "glm_moe_hidden_layout_of")
    return lay


def dense_workspace_size(T: int, D: int, F: int, dtype: torch.dtype = torch.bfloat16,
                         opts: Optional[Options] = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().glm_moe_dense_workspace_size(ctypes.byref(dims(T, D, 0, 0, F, dtype)),
                                              None if opts is None else ctypes.byref(opts),
                                              ctypes.byref(n)), "glm_moe_dense_workspace_size")
    return n.value


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def new_workspace(T, D, E, F, Fs, top_k, dtype, device=None,
                  opts: Optional[Options] = None, weight: Optional[int] = None) -> torch.Tensor:
    n = workspace_size(T, D, E, F, Fs, top_k, dtype, opts, weight)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device or "cuda")


def route(x: torch.Tensor, router_w: torch.Tensor, corr_bias: torch.Tensor, top_k: int,
          scale: float, workspace: Optional[torch.Tensor] = None,
          topk_idx: Optional[torch.Tensor] = None,
          topk_w: Optional[torch.Tensor] = None, *, n_group: int = 1, topk_group: int = 1,
          group_topk: int = 0, norm_weight: Optional[torch.Tensor] = None,
          norm_eps: float = 1e-5) -> Tuple[torch.Tensor, torch.Tensor]:
    """Router only; returns (topk_idx [T, k] int32, topk_w [T, k] float32)."""
    T, D = x.shape
    E = router_w.shape[0]
    d = dims(T, D, E, 64, 64, x.dtype)
    o = options(n_group, topk_group, group_topk, norm_weight, norm_eps, False, D)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(T, D, E, 64, 64, top_k, x.dtype, x.device, o)
    st = lib().glm_moe_route_ex(
        ctypes.byref(d), ctypes.byref(o), _ptr(x, "x"),
        _ptr(router_w, "router_w", torch.float32, (E, D)),
        _ptr(corr_bias, "corr_bias", torch.float32, (E,)), top_k, float(scale),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, top_k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, top_k)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream())
    _check(st, "glm_moe_route_ex")
    return topk_idx, topk_w


class Trace:
    """Per-stage HIP event timing of forward calls on the current stream."""

    def __init__(self, max_calls: int = 256):
        h = ctypes.c_void_p()
        _check(lib().glm_moe_trace_create(ctypes.byref(h), max_calls), "glm_moe_trace_create")
        self.handle = h

    def reset(self) -> None:
        _check(lib().glm_moe_trace_reset(self.handle), "glm_moe_trace_reset")

    def read(self) -> Tuple[dict, int]:
        """(summed milliseconds per stage, number of calls recorded)."""
        ms = (ctypes.c_float * len(STAGES))()
        n = ctypes.c_int(0)
        _check(lib().glm_moe_trace_read(self.handle, ms, ctypes.byref(n)), "glm_moe_trace_read")
        return {s: float(ms[i]) for i, s in enumerate(STAGES)}, n.value

    def close(self) -> None:
        if self.handle:
            lib().glm_moe_trace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward(x: torch.Tensor, router_w: torch.Tensor, corr_bias: torch.Tensor,
            w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
            shared_w1: torch.Tensor, shared_w3: torch.Tensor, shared_w2: torch.Tensor,
            top_k: int, scale: float, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
            trace: Optional[Trace] = None, *, n_group: int = 1, topk_group: int = 1,
            group_topk: int = 0, norm_weight: Optional[torch.Tensor] = None,
            norm_eps: float = 1e-5, residual: bool = False) -> torch.Tensor:
    """The whole MoE layer; returns ``out`` [T, D] float32.

    Pass ``topk_idx`` / ``topk_w`` tensors to also receive the routing.  With
    ``norm_weight`` the layer runs on RMSNorm(x); ``residual`` adds x to the
    output; ``n_group`` > 1 turns on group-limited routing.
    """
    T, D = x.shape
    E, F, _ = w1.shape
    Fs = shared_w1.shape[0]
    dt = x.dtype
    d = dims(T, D, E, F, Fs, dt)
    o = options(n_group, topk_group, group_topk, norm_weight, norm_eps, residual, D)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(T, D, E, F, Fs, top_k, dt, x.device, o)
    st = lib().glm_moe_forward_ex(
        ctypes.byref(d), ctypes.byref(o), _ptr(x, "x", dt, (T, D)),
        _ptr(router_w, "router_w", torch.float32, (E, D)),
        _ptr(corr_bias, "corr_bias", torch.float32, (E,)),
        _ptr(w1, "w1", dt, (E, F, D)), _ptr(w3, "w3", dt, (E, F, D)),
        _ptr(w2, "w2", dt, (E, D, F)),
        _ptr(shared_w1, "shared_w1", dt, (Fs, D)), _ptr(shared_w3, "shared_w3", dt, (Fs, D)),
        _ptr(shared_w2, "shared_w2", dt, (D, Fs)),
        top_k, float(scale), _ptr(out, "out", torch.float32, (T, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, top_k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, top_k)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(),
        None if trace is None else trace.handle)
    _check(st, "glm_moe_forward_ex")
    return out


def forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, corr_bias: torch.Tensor,
                    w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
                    shared_w1: torch.Tensor, shared_w3: torch.Tensor, shared_w2: torch.Tensor,
                    top_k: int, scale: float, out: torch.Tensor,
                    topk_idx: Optional[torch.Tensor] = None,
                    topk_w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``glm_moe_forward_noalloc``: the layer in the library's fixed per-GPU
    workspace (no allocation; ``out`` must be given)."""
    T, D = x.shape
    E, F, _ = w1.shape
    Fs = shared_w1.shape[0]
    dt = x.dtype
    st = lib().glm_moe_forward_noalloc(
        ctypes.byref(dims(T, D, E, F, Fs, dt)), _ptr(x, "x", dt, (T, D)),
        _ptr(router_w, "router_w", torch.float32, (E, D)),
        _ptr(corr_bias, "corr_bias", torch.float32, (E,)),
        _ptr(w1, "w1", dt, (E, F, D)), _ptr(w3, "w3", dt, (E, F, D)),
        _ptr(w2, "w2", dt, (E, D, F)),
        _ptr(shared_w1, "shared_w1", dt, (Fs, D)), _ptr(shared_w3, "shared_w3", dt, (Fs, D)),
        _ptr(shared_w2, "shared_w2", dt, (D, Fs)),
        top_k, float(scale), _ptr(out, "out", torch.float32, (T, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, top_k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, top_k)), _stream())
    _check(st, "glm_moe_forward_noalloc")
    return out


def dense_ffn(x: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, *,
              norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-5,
              residual: bool = False, trace: Optional[Trace] = None) -> torch.Tensor:
    """A dense SiLU-gated FFN on the same kernels; returns ``out`` [T, D] float32."""
    T, D = x.shape
    F = w1.shape[0]
    dt = x.dtype
    d = dims(T, D, 0, 0, F, dt)
    o = options(1, 1, 0, norm_weight, norm_eps, residual, D)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(dense_workspace_size(T, D, F, dt, o), 1), dtype=torch.uint8,
                                device=x.device)
    st = lib().glm_moe_dense_ffn(
        ctypes.byref(d), ctypes.byref(o), _ptr(x, "x", dt, (T, D)),
        _ptr(w1, "w1", dt, (F, D)), _ptr(w3, "w3", dt, (F, D)), _ptr(w2, "w2", dt, (D, F)),
        _ptr(out, "out", torch.float32, (T, D)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(),
        None if trace is None else trace.handle)
    _check(st, "glm_moe_dense_ffn")
    return out


def pack_mx_scales(scales: torch.Tensor) -> torch.Tensor:
    """Row-major MX scales [..., N, K/32] (uint8, on the GPU) -> the
    K-step-major layout [..., K/128, N, 4] that ``forward_mx`` takes."""
    if scales.dim() < 2:
        raise ValueError("scales must be [..., N, K/32]")
    *lead, N, KS = scales.shape
    n_mats = 1
    for v in lead:
        n_mats *= v
    out = torch.empty((*lead, KS // 4, N, 4), dtype=torch.uint8, device=scales.device)
    st = lib().glm_moe_mx_pack_scales(_ptr(scales, "scales", torch.uint8), _ptr(out, "out"),
                                      n_mats, N, KS * 32, _stream())
    _check(st, "glm_moe_mx_pack_scales")
    return out


def forward_mx(x: torch.Tensor, router_w: torch.Tensor, corr_bias: torch.Tensor,
               w1: torch.Tensor, w1_scale: torch.Tensor, w3: torch.Tensor,
               w3_scale: torch.Tensor, w2: torch.Tensor, w2_scale: torch.Tensor,
               shared_w1: torch.Tensor, shared_w1_scale: torch.Tensor,
               shared_w3: torch.Tensor, shared_w3_scale: torch.Tensor,
               shared_w2: torch.Tensor, shared_w2_scale: torch.Tensor,
               top_k: int, scale: float, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None,
               topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
               trace: Optional[Trace] = None, *, n_group: int = 1, topk_group: int = 1,
               group_topk: int = 0, norm_weight: Optional[torch.Tensor] = None,
               norm_eps: float = 1e-5, residual: bool = False) -> torch.Tensor:
    """The layer with MXFP8 expert weights (uint8 E4M3 codes and uint8 E8M0
    scales, one per 32 elements along each row, in the K-step-major layout of
    ``pack_mx_scales``); x is bfloat16."""
    T, D = x.shape
    E, F, _ = w1.shape
    Fs = shared_w1.shape[0]
    u8 = torch.uint8
    d = dims(T, D, E, F, Fs, x.dtype, MXFP8)
    o = options(n_group, topk_group, group_topk, norm_weight, norm_eps, residual, D)
    W = MxWeights(
        _ptr(w1, "w1", u8, (E, F, D)), _ptr(w1_scale, "w1_scale", u8, (E, D // 128, F, 4)),
        _ptr(w3, "w3", u8, (E, F, D)), _ptr(w3_scale, "w3_scale", u8, (E, D // 128, F, 4)),
        _ptr(w2, "w2", u8, (E, D, F)), _ptr(w2_scale, "w2_scale", u8, (E, F // 128, D, 4)),
        _ptr(shared_w1, "shared_w1", u8, (Fs, D)),
        _ptr(shared_w1_scale, "shared_w1_scale", u8, (D // 128, Fs, 4)),
        _ptr(shared_w3, "shared_w3", u8, (Fs, D)),
        _ptr(shared_w3_scale, "shared_w3_scale", u8, (D // 128, Fs, 4)),
        _ptr(shared_w2, "shared_w2", u8, (D, Fs)),
        _ptr(shared_w2_scale, "shared_w2_scale", u8, (Fs // 128, D, 4)))
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(T, D, E, F, Fs, top_k, x.dtype, x.device, o, MXFP8)
    st = lib().glm_moe_forward_mx(
        ctypes.byref(d), ctypes.byref(o), _ptr(x, "x", torch.bfloat16, (T, D)),
        _ptr(router_w, "router_w", torch.float32, (E, D)),
        _ptr(corr_bias, "corr_bias", torch.float32, (E,)), ctypes.byref(W), top_k,
        float(scale), _ptr(out, "out", torch.float32, (T, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, top_k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, top_k)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(),
        None if trace is None else trace.handle)
    _check(st, "glm_moe_forward_mx")
    return out
