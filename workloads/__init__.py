"""Seeded synthetic inputs for the GLM-5.2 mixture-of-experts feed-forward layer.

This module is shared by the CPU oracle and by the GPU path (tests and bench).
It only draws numbers and encodes them; it performs none of the layer's
arithmetic.  bf16 tensors are returned as ``numpy.uint16`` bit patterns
(round-to-nearest-even from an fp32 draw); each consumer decodes them itself.

Shapes follow the GLM-5.2 anatomy pages: hidden 6144, 256 routed experts with
8 active per token, expert width 2048, one shared expert, routed scale 2.5
(frontier-model-atlas "GLM-5.2 model anatomy", Feed-forward / Mixture of
Experts panel; PocketLLM "GLM-5.2" Model specification table).

Recipe (every stream is independent and addressable):

* stream ids: ``SeedSequence([seed, tensor_id, expert_id])``;
  tensor ids 0 x, 1 router_w, 2 corr_bias, 3 w1, 4 w3, 5 w2, 6 shared_w1,
  7 shared_w3, 8 shared_w2, 9 norm_weight, 10 residual stream h, 11-13 the
  dense FFN's w1, w3, w2.
* draws: ``standard_normal(float32) * float32(std)``; bf16 tensors are the
  RNE rounding of that fp32 value.
* x ~ N(0, 1); router_w ~ N(0, 1/D); w1, w3 ~ N(0, 1/D); w2 ~ N(0, 1/F);
  shared likewise with F_s.  (The variance reading of ``N(0, 1/fan_in)``.)
* corr_bias ~ N(0, bias_std) (the std reading); the skewed workloads then set
  the first ``hot_count`` entries to ``hot_value``.
* Pre-norm block: h ~ N(0, 3^2) (a residual stream larger than unit scale, so
  the norm is not near the identity); norm_weight = 1 + N(0, 0.1^2).
* Dense FFN of width F_d: w1, w3 ~ N(0, 1/D), w2 ~ N(0, 1/F_d).
* The layer weights (router, routed and shared experts) are seeded by
  ``weight_seed``; the GLM-shape workloads share one weight set, i.e. one
  layer seen with different token batches and bias regimes.  ``x`` and
  ``corr_bias`` are seeded by the workload's own ``seed``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, Optional, Tuple

import numpy as np

(TID_X, TID_RW, TID_BIAS, TID_W1, TID_W3, TID_W2, TID_SW1, TID_SW3, TID_SW2, TID_NORM, TID_H,
 TID_DW1, TID_DW3, TID_DW2) = range(14)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    E: int
    k: int
    F: int
    Fs: int
    dtype: str  # "f32", "bf16" (activations and weights), "mxfp8" (bf16 activations,
                #  MXFP8 expert weights)
    scale: float
    bias_std: float
    seed: int
    weight_seed: int
    hot_count: int = 0
    hot_value: float = 0.0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


GLM_WEIGHT_SEED = 1000
# Width of the leading dense FFN layers.  The pages give the count (three) but
# not the width; this stand-in is 9 x 2048, the routed plus shared width one
# token passes through in a MoE layer, so a dense layer does the same work per
# token.
GLM_DENSE_WIDTH = 18432

WORKLOADS = {
    # tiny fp32 layer (parity at 1e-5)
    "tiny_f32": Workload("tiny_f32", T=64, D=128, E=8, k=2, F=64, Fs=64, dtype="f32",
                         scale=2.5, bias_std=0.1, seed=1, weight_seed=1),
    # mid-size bf16 layer
    "mid_bf16": Workload("mid_bf16", T=512, D=1024, E=64, k=4, F=512, Fs=512, dtype="bf16",
                         scale=2.5, bias_std=0.1, seed=2, weight_seed=2),
    # mid-size layer with MXFP8 expert weights (bf16 activations)
    "mid_mx": Workload("mid_mx", T=512, D=1024, E=64, k=4, F=512, Fs=512, dtype="mxfp8",
                       scale=2.5, bias_std=0.1, seed=2, weight_seed=2),
    # GLM-5.2 shape, 64-token decode step
    "glm_decode": Workload("glm_decode", T=64, D=6144, E=256, k=8, F=2048, Fs=2048, dtype="bf16",
                           scale=2.5, bias_std=0.1, seed=3, weight_seed=GLM_WEIGHT_SEED),
    # GLM-5.2 shape, 8192-token prefill chunk, near-uniform routing
    "glm_prefill": Workload("glm_prefill", T=8192, D=6144, E=256, k=8, F=2048, Fs=2048,
                            dtype="bf16", scale=2.5, bias_std=0.01, seed=4,
                            weight_seed=GLM_WEIGHT_SEED),
    # GLM-5.2 shape, 2048-token chunk (about 64 rows per expert: middle tiles)
    "glm_chunk_2k": Workload("glm_chunk_2k", T=2048, D=6144, E=256, k=8, F=2048, Fs=2048,
                             dtype="bf16", scale=2.5, bias_std=0.01, seed=6,
                             weight_seed=GLM_WEIGHT_SEED),
    # GLM-5.2 shape, 4096 tokens, +1.5 bias on experts 0..15 (literal skew)
    "glm_skew": Workload("glm_skew", T=4096, D=6144, E=256, k=8, F=2048, Fs=2048, dtype="bf16",
                         scale=2.5, bias_std=0.05, seed=5, weight_seed=GLM_WEIGHT_SEED,
                         hot_count=16, hot_value=1.5),
    # GLM-5.2 shape, 4096 tokens, milder hot bias (+0.2) on experts 0..15
    "glm_skew_mild": Workload("glm_skew_mild", T=4096, D=6144, E=256, k=8, F=2048, Fs=2048,
                              dtype="bf16", scale=2.5, bias_std=0.05, seed=55,
                              weight_seed=GLM_WEIGHT_SEED, hot_count=16, hot_value=0.2),
    # the GLM-5.2 decode and prefill batches with MXFP8 expert weights (the same
    # fp32 draws, encoded as MXFP8 instead of bf16)
    "glm_decode_mx": Workload("glm_decode_mx", T=64, D=6144, E=256, k=8, F=2048, Fs=2048,
                              dtype="mxfp8", scale=2.5, bias_std=0.1, seed=3,
                              weight_seed=GLM_WEIGHT_SEED),
    "glm_prefill_mx": Workload("glm_prefill_mx", T=8192, D=6144, E=256, k=8, F=2048, Fs=2048,
                               dtype="mxfp8", scale=2.5, bias_std=0.01, seed=4,
                               weight_seed=GLM_WEIGHT_SEED),
}


def _rng(seed: int, tensor_id: int, expert_id: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, expert_id]))


def normal_f32(seed: int, tensor_id: int, expert_id: int, shape, std: float) -> np.ndarray:
    """fp32 draws ``N(0, std^2)`` from one addressable stream."""
    n = int(np.prod(shape))
    a = _rng(seed, tensor_id, expert_id).standard_normal(n, dtype=np.float32)
    a *= np.float32(std)
    return a.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite (normal draws), so no NaN special case is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = u >> np.uint32(16)
    b &= np.uint32(1)
    b += np.uint32(0x7FFF)
    b += u
    b >>= np.uint32(16)
    return b.astype(np.uint16)


def f32_to_mxfp8(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Encode fp32 values as OCP MXFP8 along the last axis (blocks of 32).

    Returns (E4M3 codes uint8, E8M0 scales uint8 [..., n/32]).  Block scale:
    the smallest 2^s with max|v| <= 448 * 2^s; elements v * 2^-s rounded to the
    nearest E4M3 value, ties to even (integer rounding of the fp32 bit pattern
    for normal results, of v * 2^9 for results below 2^-6).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    n = a.shape[-1]
    assert n % 32 == 0, "MXFP8 rows must be a multiple of 32 long"
    blk = a.reshape(a.shape[:-1] + (n // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    mant, ex = np.frexp(amax)                          # amax = mant * 2^ex
    s = np.where(mant <= np.float32(0.875), ex - 9, ex - 8)
    s = np.where(amax == 0, 0, s).astype(np.int32)
    y = np.ldexp(blk, -s[..., None]).astype(np.float32)  # exact power-of-two scaling
    mag = np.abs(y)
    u = mag.view(np.uint32).astype(np.int64)
    normal = (u >> 23) >= (127 - 6)
    rn = (u + 0x7FFFF + ((u >> 20) & 1)) >> 20         # 8-bit exponent, 3-bit mantissa
    code = np.where(normal, rn - ((127 - 7) << 3), np.rint(mag * np.float32(512.0)))
    code = code.astype(np.int64) | np.where(np.signbit(y) & (mag > 0), 0x80, 0)
    return code.astype(np.uint8).reshape(a.shape), (s + 127).astype(np.uint8)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Activations (and f32/bf16 weights) in the workload's storage format."""
    return a if dtype == "f32" else f32_to_bf16_bits(a)


def _encode_weight(a: np.ndarray, dtype: str):
    """Expert weights: as ``_encode``, or an (codes, scales) pair for MXFP8."""
    return f32_to_mxfp8(a) if dtype == "mxfp8" else _encode(a, dtype)


# ---------------------------------------------------------------- per tensor

def make_x(w: Workload, T: Optional[int] = None) -> np.ndarray:
    T = w.T if T is None else T
    return _encode(normal_f32(w.seed, TID_X, 0, (T, w.D), 1.0), w.dtype)


def make_router_w(w: Workload) -> np.ndarray:
    """fp32 [E, D]."""
    return normal_f32(w.weight_seed, TID_RW, 0, (w.E, w.D), 1.0 / np.sqrt(w.D))


def make_corr_bias(w: Workload) -> np.ndarray:
    """fp32 [E]."""
    b = normal_f32(w.seed, TID_BIAS, 0, (w.E,), w.bias_std)
    if w.hot_count:
        b[: w.hot_count] = np.float32(w.hot_value)
    return b


def make_expert(w: Workload, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(w1 [F, D], w3 [F, D], w2 [D, F]) of routed expert ``e`` in the workload dtype."""
    s_in, s_out = 1.0 / np.sqrt(w.D), 1.0 / np.sqrt(w.F)
    w1 = normal_f32(w.weight_seed, TID_W1, e, (w.F, w.D), s_in)
    w3 = normal_f32(w.weight_seed, TID_W3, e, (w.F, w.D), s_in)
    w2 = normal_f32(w.weight_seed, TID_W2, e, (w.D, w.F), s_out)
    return _encode_weight(w1, w.dtype), _encode_weight(w3, w.dtype), _encode_weight(w2, w.dtype)


def make_shared(w: Workload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(shared_w1 [Fs, D], shared_w3 [Fs, D], shared_w2 [D, Fs])."""
    s_in, s_out = 1.0 / np.sqrt(w.D), 1.0 / np.sqrt(w.Fs)
    w1 = normal_f32(w.weight_seed, TID_SW1, 0, (w.Fs, w.D), s_in)
    w3 = normal_f32(w.weight_seed, TID_SW3, 0, (w.Fs, w.D), s_in)
    w2 = normal_f32(w.weight_seed, TID_SW2, 0, (w.D, w.Fs), s_out)
    return _encode_weight(w1, w.dtype), _encode_weight(w3, w.dtype), _encode_weight(w2, w.dtype)


def make_norm_weight(w: Workload) -> np.ndarray:
    """fp32 [D]: RMSNorm weight of the block, 1 + N(0, 0.1^2)."""
    return (np.float32(1.0) + normal_f32(w.weight_seed, TID_NORM, 0, (w.D,), 0.1)).astype(
        np.float32)


def make_hidden(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Residual stream h [T, D] ~ N(0, 9) in the activation dtype."""
    T = w.T if T is None else T
    return _encode(normal_f32(w.seed, TID_H, 0, (T, w.D), 3.0), w.dtype)


def make_dense(w: Workload, F: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(w1 [F, D], w3 [F, D], w2 [D, F]) of a dense SiLU-gated FFN of width F."""
    s_in, s_out = 1.0 / np.sqrt(w.D), 1.0 / np.sqrt(F)
    w1 = normal_f32(w.weight_seed, TID_DW1, 0, (F, w.D), s_in)
    w3 = normal_f32(w.weight_seed, TID_DW3, 0, (F, w.D), s_in)
    w2 = normal_f32(w.weight_seed, TID_DW2, 0, (w.D, F), s_out)
    return _encode(w1, w.dtype), _encode(w3, w.dtype), _encode(w2, w.dtype)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_experts(w: Workload, threads: Optional[int] = None,
                 experts=None) -> Iterator[Tuple[int, Tuple[np.ndarray, np.ndarray, np.ndarray]]]:
    """Yield ``(e, make_expert(w, e))`` in expert order, drawn by a thread pool.

    At most ``2 * threads`` experts are held at once, so the GLM-shape weight
    set (19.3 GB of bf16) can be streamed to the device without a host copy.
    """
    threads = threads or default_threads()
    experts = list(range(w.E)) if experts is None else list(experts)
    with ThreadPoolExecutor(threads) as ex:
        window = []
        it = iter(experts)
        for e in it:
            window.append((e, ex.submit(make_expert, w, e)))
            if len(window) >= 2 * threads:
                e0, f0 = window.pop(0)
                yield e0, f0.result()
        for e0, f0 in window:
            yield e0, f0.result()


@dataclasses.dataclass
class HostLayer:
    """All inputs of one layer call, host side (bf16 as uint16 bits)."""
    w: Workload
    x: np.ndarray
    router_w: np.ndarray
    corr_bias: np.ndarray
    w1: np.ndarray  # [E, F, D]
    w3: np.ndarray  # [E, F, D]
    w2: np.ndarray  # [E, D, F]
    sw1: np.ndarray
    sw3: np.ndarray
    sw2: np.ndarray
    # MXFP8 weights: the fields above hold E4M3 codes, these the E8M0 scales
    # (one per 32 elements along each row)
    w1s: Optional[np.ndarray] = None  # [E, F, D/32]
    w3s: Optional[np.ndarray] = None
    w2s: Optional[np.ndarray] = None  # [E, D, F/32]
    sw1s: Optional[np.ndarray] = None
    sw3s: Optional[np.ndarray] = None
    sw2s: Optional[np.ndarray] = None

    def expert(self, e: int):
        """Expert e's weights: (w1, w3, w2), or ((codes, scales) x 3) for MXFP8."""
        if self.w1s is None:
            return self.w1[e], self.w3[e], self.w2[e]
        return ((self.w1[e], self.w1s[e]), (self.w3[e], self.w3s[e]), (self.w2[e], self.w2s[e]))

    def shared(self):
        if self.sw1s is None:
            return self.sw1, self.sw3, self.sw2
        return ((self.sw1, self.sw1s), (self.sw3, self.sw3s), (self.sw2, self.sw2s))


def make_layer(w: Workload, threads: Optional[int] = None) -> HostLayer:
    """Whole layer on the host (use for sizes that fit comfortably in RAM)."""
    x, rw, cb = make_x(w), make_router_w(w), make_corr_bias(w)
    if w.dtype == "mxfp8":
        w1 = np.empty((w.E, w.F, w.D), np.uint8)
        w3 = np.empty((w.E, w.F, w.D), np.uint8)
        w2 = np.empty((w.E, w.D, w.F), np.uint8)
        w1s = np.empty((w.E, w.F, w.D // 32), np.uint8)
        w3s = np.empty((w.E, w.F, w.D // 32), np.uint8)
        w2s = np.empty((w.E, w.D, w.F // 32), np.uint8)
        for e, (a, b, c) in iter_experts(w, threads):
            (w1[e], w1s[e]), (w3[e], w3s[e]), (w2[e], w2s[e]) = a, b, c
        (sw1, sw1s), (sw3, sw3s), (sw2, sw2s) = make_shared(w)
        return HostLayer(w, x, rw, cb, w1, w3, w2, sw1, sw3, sw2, w1s, w3s, w2s, sw1s, sw3s,
                         sw2s)
    et = np.float32 if w.dtype == "f32" else np.uint16
    w1 = np.empty((w.E, w.F, w.D), et)
    w3 = np.empty((w.E, w.F, w.D), et)
    w2 = np.empty((w.E, w.D, w.F), et)
    for e, (a, b, c) in iter_experts(w, threads):
        w1[e], w3[e], w2[e] = a, b, c
    sw1, sw3, sw2 = make_shared(w)
    return HostLayer(w, x, rw, cb, w1, w3, w2, sw1, sw3, sw2)
