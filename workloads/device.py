"""Upload seeded layer inputs to the GPU with PyTorch (memory plumbing only).

Used by the GPU tests and the benchmark.  bf16 bit patterns (uint16) become
``torch.bfloat16`` tensors with identical bits.
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

    def args(self):
        return (self.x, self.router_w, self.corr_bias, self.w1, self.w3, self.w2,
                self.sw1, self.sw3, self.sw2)


def upload_layer(L: HostLayer, device="cuda") -> DeviceLayer:
    return DeviceLayer(L.w, to_device(L.x, device), to_device(L.router_w, device),
                       to_device(L.corr_bias, device), to_device(L.w1, device),
                       to_device(L.w3, device), to_device(L.w2, device),
                       to_device(L.sw1, device), to_device(L.sw3, device),
                       to_device(L.sw2, device))


def stream_layer(w: Workload, device="cuda", keep_host: bool = False,
                 threads: Optional[int] = None):
    """Draw the layer expert by expert straight into device tensors.

    Returns ``(DeviceLayer, HostLayer or None)``; with ``keep_host`` the host
    copy (bf16 bits) is kept for the oracle.
    """
    dt = torch_dtype(w)
    w1 = torch.empty((w.E, w.F, w.D), dtype=dt, device=device)
    w3 = torch.empty((w.E, w.F, w.D), dtype=dt, device=device)
    w2 = torch.empty((w.E, w.D, w.F), dtype=dt, device=device)
    host = None
    if keep_host:
        et = np.float32 if w.dtype == "f32" else np.uint16
        hw1 = np.empty((w.E, w.F, w.D), et)
        hw3 = np.empty((w.E, w.F, w.D), et)
        hw2 = np.empty((w.E, w.D, w.F), et)
    for e, (a, b, c) in iter_experts(w, threads):
        w1[e].copy_(to_device(a, "cpu"))
        w3[e].copy_(to_device(b, "cpu"))
        w2[e].copy_(to_device(c, "cpu"))
        if keep_host:
            hw1[e], hw3[e], hw2[e] = a, b, c
    sw1, sw3, sw2 = make_shared(w)
    x, rw, cb = make_x(w), make_router_w(w), make_corr_bias(w)
    dev = DeviceLayer(w, to_device(x, device), to_device(rw, device), to_device(cb, device),
                      w1, w3, w2, to_device(sw1, device), to_device(sw3, device),
                      to_device(sw2, device))
    if keep_host:
        host = HostLayer(w, x, rw, cb, hw1, hw3, hw2, sw1, sw3, sw2)
    torch.cuda.synchronize()
    return dev, host
