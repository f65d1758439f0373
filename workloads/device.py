"""Upload seeded layer inputs to the GPU with PyTorch (memory plumbing only).

Used by the GPU tests and the benchmark.  bf16 bit patterns (uint16) become
``torch.bfloat16`` tensors with identical bits; MXFP8 scales, generated
row-major [..., N, K/32], are handed over in the K-step-major layout
[..., K/128, N, 4] the layer takes (a byte permutation).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import HostLayer, Workload, iter_experts, make_corr_bias, make_router_w, make_shared, make_x


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def kstep_major(scales: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """Row-major MX scales [..., N, K/32] -> [..., K/128, N, 4]."""
    if scales is None:
        return None
    *lead, n, ks = scales.shape
    return scales.reshape(*lead, n, ks // 4, 4).transpose(-3, -2).contiguous()


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


@dataclasses.dataclass
class DeviceLayer:
    w: Workload
    x: torch.Tensor
    router_w: torch.Tensor
    corr_bias: torch.Tensor
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    sw1: torch.Tensor
    sw3: torch.Tensor
    sw2: torch.Tensor

    # MXFP8 scales (None for f32 / bf16 weights)
    w1s: Optional[torch.Tensor] = None
    w3s: Optional[torch.Tensor] = None
    w2s: Optional[torch.Tensor] = None
    sw1s: Optional[torch.Tensor] = None
    sw3s: Optional[torch.Tensor] = None
    sw2s: Optional[torch.Tensor] = None

    def args(self):
        """Positional tensor arguments of ``forward`` (or ``forward_mx``)."""
        if self.w1s is None:
            return (self.x, self.router_w, self.corr_bias, self.w1, self.w3, self.w2,
                    self.sw1, self.sw3, self.sw2)
        return (self.x, self.router_w, self.corr_bias, self.w1, self.w1s, self.w3, self.w3s,
                self.w2, self.w2s, self.sw1, self.sw1s, self.sw3, self.sw3s, self.sw2, self.sw2s)

    def with_x(self, x: torch.Tensor, corr_bias: Optional[torch.Tensor] = None,
               w: Optional[Workload] = None) -> "DeviceLayer":
        """The same weights with another input batch (and bias)."""
        return dataclasses.replace(self, x=x, w=self.w if w is None else w,
                                   corr_bias=self.corr_bias if corr_bias is None else corr_bias)


def upload_layer(L: HostLayer, device="cuda") -> DeviceLayer:
    t = lambda a: None if a is None else to_device(a, device)
    s = lambda a: kstep_major(t(a))
    return DeviceLayer(L.w, t(L.x), t(L.router_w), t(L.corr_bias), t(L.w1), t(L.w3), t(L.w2),
                       t(L.sw1), t(L.sw3), t(L.sw2), s(L.w1s), s(L.w3s), s(L.w2s), s(L.sw1s),
                       s(L.sw3s), s(L.sw2s))


def stream_layer(w: Workload, device="cuda", keep_host: bool = False,
                 threads: Optional[int] = None):
    """Draw the layer expert by expert straight into device tensors.

    Returns ``(DeviceLayer, HostLayer or None)``; with ``keep_host`` the host
    copy (bf16 bits, or MXFP8 codes and scales) is kept for the oracle.
    """
    mx = w.dtype == "mxfp8"
    dt = torch.uint8 if mx else torch_dtype(w)
    et = np.uint8 if mx else (np.float32 if w.dtype == "f32" else np.uint16)
    shapes = {"w1": (w.E, w.F, w.D), "w3": (w.E, w.F, w.D), "w2": (w.E, w.D, w.F)}
    if mx:
        shapes.update(w1s=(w.E, w.F, w.D // 32), w3s=(w.E, w.F, w.D // 32),
                      w2s=(w.E, w.D, w.F // 32))
    dev_t = {k: torch.empty(v, dtype=dt, device=device) for k, v in shapes.items()}
    host_t = {k: np.empty(v, et) for k, v in shapes.items()} if keep_host else None
    for e, parts in iter_experts(w, threads):
        if mx:
            (a, a_s), (b, b_s), (c, c_s) = parts
            vals = dict(w1=a, w3=b, w2=c, w1s=a_s, w3s=b_s, w2s=c_s)
        else:
            vals = dict(zip(("w1", "w3", "w2"), parts))
        for k, v in vals.items():
            dev_t[k][e].copy_(to_device(v, "cpu"))
            if keep_host:
                host_t[k][e] = v
    sh = make_shared(w)
    x, rw, cb = make_x(w), make_router_w(w), make_corr_bias(w)
    if mx:
        (sw1, sw1s), (sw3, sw3s), (sw2, sw2s) = sh
        sc = [sw1s, sw3s, sw2s]
    else:
        sw1, sw3, sw2 = sh
        sc = [None, None, None]
    t = lambda a: None if a is None else to_device(a, device)
    s = lambda a: kstep_major(t(a))
    dev = DeviceLayer(w, t(x), t(rw), t(cb), dev_t["w1"], dev_t["w3"], dev_t["w2"], t(sw1),
                      t(sw3), t(sw2), kstep_major(dev_t.get("w1s")), kstep_major(dev_t.get("w3s")),
                      kstep_major(dev_t.get("w2s")), s(sc[0]), s(sc[1]), s(sc[2]))
    host = None
    if keep_host:
        host = HostLayer(w, x, rw, cb, host_t["w1"], host_t["w3"], host_t["w2"], sw1, sw3, sw2,
                         host_t.get("w1s"), host_t.get("w3s"), host_t.get("w2s"), *sc)
    torch.cuda.synchronize()
    return dev, host
