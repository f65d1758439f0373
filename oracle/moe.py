"""CPU float64 oracle of the GLM-5.2 mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP path: it decodes its own inputs, and every step is written out plainly
in float64 NumPy, in the order the layer is stated.

The layer (frontier-model-atlas "GLM-5.2 model anatomy", Feed-forward / Mixture
of Experts panel): sigmoid router scores over 256 routed experts; an
expert-score correction bias takes part in the top-8 selection only; the
selected *un-biased* scores are renormalised and scaled by 2.5; the expert
outputs are then merged with one always-on shared expert.  Expert MLPs use the
w1 / w3 / w2 roles named on the PocketLLM "GLM-5.2" page (Implemented execution
path): SiLU(x w1^T) * (x w3^T), then w2.

Readings taken where the pages are silent (each also listed in the design doc):

* the bias is added to the post-sigmoid score, not to the logit;
* one expert group (plain top-k over all experts);
* renormalisation divides by the sum of the k selected un-biased scores, no eps;
* the shared expert carries weight 1 (only routed weights are scaled);
* ties in the biased score go to the lower expert index; slots are ordered by
  descending biased score;
* dropless: every (token, slot) assignment is computed.

Parity pins: tests/test_oracle_pins.py (sum of weights, bias-moves-selection,
brute-force top-k, identity-expert closed form, shared-only, invariances).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

from . import mx

Expert = Tuple[np.ndarray, np.ndarray, np.ndarray]


# ----------------------------------------------------------------- decoding

def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the high half of an IEEE fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode(a: np.ndarray) -> np.ndarray:
    """float64 value of an input tensor: uint16 means bf16 bits, else its own value."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ------------------------------------------------------------------ routing

def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def select_topk(beta: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest biased scores per row.

    Order: descending score; equal scores keep ascending expert index (a stable
    sort of -beta).  -0.0 and +0.0 compare equal, so they tie.
    """
    order = np.argsort(-beta, axis=-1, kind="stable")
    return order[..., :k]


def select_topk_grouped(beta: np.ndarray, k: int, n_group: int, topk_group: int,
                        group_topk: int = 2) -> np.ndarray:
    """Group-limited top-k.

    Experts form ``n_group`` consecutive groups.  A group's score is the sum of
    its ``group_topk`` largest biased scores; each token keeps the
    ``topk_group`` best groups (equal scores: lower group index), and the k
    experts are then the top-k of the biased scores inside the kept groups
    (same order and tie rule as ``select_topk``).  ``n_group == 1`` is plain
    top-k.
    """
    T, E = beta.shape
    if n_group <= 1:
        return select_topk(beta, k)
    gs = E // n_group
    grouped = beta.reshape(T, n_group, gs)
    top_in_group = -np.sort(-grouped, axis=2)[:, :, :group_topk]
    gscore = top_in_group.sum(axis=2)
    keep = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, keep, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), beta, -np.inf)
    return select_topk(masked, k)


def group_scores(beta: np.ndarray, n_group: int, group_topk: int = 2) -> np.ndarray:
    """Per-token group scores used by ``select_topk_grouped`` ([T, n_group])."""
    T, E = beta.shape
    g = beta.reshape(T, n_group, E // n_group)
    return (-np.sort(-g, axis=2)[:, :, :group_topk]).sum(axis=2)


@dataclasses.dataclass
class Routing:
    idx: np.ndarray      # [T, k] int64, slot order
    weight: np.ndarray   # [T, k] float64
    sigma: np.ndarray    # [T, E] un-biased sigmoid scores
    beta: np.ndarray     # [T, E] biased scores used for selection


def route(x, router_w, corr_bias, top_k: int, scale: float,
          force_idx: Optional[np.ndarray] = None, n_group: int = 1, topk_group: int = 1,
          group_topk: int = 2) -> Routing:
    """Steps 1-4 of the layer.

    1. z = x W_r^T, sigma = 1 / (1 + exp(-z))           (sigmoid router scores)
    2. beta = sigma + b                                   (correction bias)
    3. idx = top_k of beta, ties to the lower index       (selection; with
       n_group > 1, only inside the token's topk_group best expert groups)
    4. w_j = (sigma[idx_j] / sum_i sigma[idx_i]) * scale  (un-biased renormalise, then x2.5)

    ``force_idx`` replaces step 3 (used to evaluate the layer on a selection
    that another implementation made at a near-tie); step 4 still runs.
    """
    x = decode(x)
    W = decode(router_w)
    b = decode(corr_bias)
    z = x @ W.T
    sigma = sigmoid(z)
    beta = sigma + b[None, :]
    if force_idx is None:
        idx = select_topk_grouped(beta, top_k, n_group, topk_group, group_topk)
    else:
        idx = np.asarray(force_idx, dtype=np.int64)
    sel = np.take_along_axis(sigma, idx, axis=1)
    weight = (sel / sel.sum(axis=1, keepdims=True)) * scale  # renormalise, then scale
    return Routing(idx=idx.astype(np.int64), weight=weight, sigma=sigma, beta=beta)


def topk_gap(beta: np.ndarray, k: int) -> np.ndarray:
    """Per-token gap between the k-th and (k+1)-th largest biased score (inf if k == E)."""
    E = beta.shape[1]
    if k >= E:
        return np.full(beta.shape[0], np.inf)
    s = -np.sort(-beta, axis=1)
    return s[:, k - 1] - s[:, k]


# ------------------------------------------------------------------ experts

def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_mlp(xr: np.ndarray, w1, w3, w2) -> np.ndarray:
    """SiLU(x w1^T) * (x w3^T), then (.) w2^T; w1, w3 are [F, D], w2 is [D, F]."""
    w1, w3, w2 = decode(w1), decode(w3), decode(w2)
    h = silu(xr @ w1.T) * (xr @ w3.T)
    return h @ w2.T


def forward(x, router_w, corr_bias,
            experts: Callable[[int], Expert],
            shared: Expert,
            top_k: int, scale: float,
            force_idx: Optional[np.ndarray] = None,
            routing: Optional[Routing] = None,
            n_group: int = 1, topk_group: int = 1,
            group_topk: int = 2) -> Tuple[np.ndarray, Routing]:
    """The whole layer: returns ``(out [T, D] float64, routing)``.

    ``experts(e)`` returns routed expert e's ``(w1, w3, w2)`` (any dtype that
    ``decode`` accepts), so the GLM-shape layer never needs all 256 experts in
    float64 at once.

    5. for every expert e: routed[t] += w[t, j] * MLP_e(x[t]) for each (t, j)
       with idx[t, j] == e
    6. out = routed + MLP_shared(x)                      (always-on shared expert)
    """
    xd = decode(x)
    r = routing if routing is not None else route(xd, router_w, corr_bias, top_k, scale, force_idx,
                                                  n_group, topk_group, group_topk)
    T, D = xd.shape
    routed = np.zeros((T, D))
    for e in np.unique(r.idx):
        tok, slot = np.nonzero(r.idx == e)
        y = expert_mlp(xd[tok], *experts(int(e)))
        routed[tok] += r.weight[tok, slot][:, None] * y
    out = routed + expert_mlp(xd, *shared)
    return out, r


def forward_arrays(x, router_w, corr_bias, w1, w3, w2, sw1, sw3, sw2,
                   top_k: int, scale: float,
                   force_idx: Optional[np.ndarray] = None) -> Tuple[np.ndarray, Routing]:
    """``forward`` with stacked expert tensors w1, w3 [E, F, D] and w2 [E, D, F]."""
    return forward(x, router_w, corr_bias, lambda e: (w1[e], w3[e], w2[e]),
                   (sw1, sw3, sw2), top_k, scale, force_idx)


def expert_load(idx: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, slot) assignments per expert (the utilisation histogram)."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=E)


# ------------------------------------------------ block around the layer

def rmsnorm(h: np.ndarray, weight, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * weight, per row."""
    h = decode(h)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * decode(weight)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float64 values (finite inputs)."""
    f = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(f)                     # f = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)  # keep 8 significant bits, ties to even
    return q


def block_ffn(h, norm_weight, eps: float, x_dtype: str, layer) -> Tuple[np.ndarray, object]:
    """The pre-norm block's feed-forward half: h + FFN(RMSNorm(h)).

    ``layer(x)`` is the feed-forward (the MoE layer or a dense MLP) and returns
    (out, extra).  The normalised input is held in the activation dtype
    (``x_dtype`` "bf16" rounds it to bf16, "f32" to fp32), as the layer
    receives it in a model of that dtype.
    """
    hd = decode(h)
    xn = rmsnorm(hd, norm_weight, eps)
    xn = round_bf16(xn) if x_dtype == "bf16" else xn.astype(np.float32).astype(np.float64)
    out, extra = layer(xn)
    return hd + out, extra


def dense_ffn(x, w1, w3, w2) -> np.ndarray:
    """A dense SiLU-gated MLP (the leading dense layers use this form)."""
    return expert_mlp(decode(x), w1, w3, w2)


# ------------------------------------------------------ MXFP8 expert variant

MxTensor = Tuple[np.ndarray, np.ndarray]        # (E4M3 codes, E8M0 scales)
MxExpert = Tuple[MxTensor, MxTensor, MxTensor]  # w1, w3, w2


def expert_hidden_mx(xq: np.ndarray, w1: MxTensor, w3: MxTensor) -> np.ndarray:
    """The gated hidden values SiLU(x w1^T) * (x w3^T) of the MXFP8 expert MLP,
    before they are quantised (``xq``: values of the quantised input rows)."""
    W1, W3 = mx.dequantize(*w1), mx.dequantize(*w3)
    return silu(xq @ W1.T) * (xq @ W3.T)


def expert_mlp_mx(xq: np.ndarray, w1: MxTensor, w3: MxTensor, w2: MxTensor) -> np.ndarray:
    """The SiLU-gated expert MLP with MXFP8 weights, on an MXFP8 input.

    ``xq`` holds the values of the already quantised input rows.  The gated
    hidden value SiLU(x w1^T) * (x w3^T) is quantised to MXFP8 along the hidden
    dimension before the w2 product, as the down projection consumes it in that
    format.
    """
    h = expert_hidden_mx(xq, w1, w3)
    return mx.fake_quantize(h) @ mx.dequantize(*w2).T


def forward_mx_on_hidden(routing: Routing, hidden: np.ndarray, shared_hidden: np.ndarray,
                         experts: Callable[[int], MxExpert], shared: MxExpert) -> np.ndarray:
    """Steps 5-6 of the MXFP8 layer from given quantised hidden values.

    ``hidden[t, j]`` holds the values of token t's quantised gated hidden row
    for slot j (expert ``routing.idx[t, j]``), ``shared_hidden[t]`` the shared
    expert's.  Returns out[t] = sum_j w[t, j] (hidden[t, j] w2_e^T)
    + shared_hidden[t] w2_shared^T.
    """
    T, k, _ = hidden.shape
    D = mx.dequantize(*shared[2]).shape[0]
    routed = np.zeros((T, D))
    for e in np.unique(routing.idx):
        tok, slot = np.nonzero(routing.idx == e)
        y = hidden[tok, slot] @ mx.dequantize(*experts(int(e))[2]).T
        routed[tok] += routing.weight[tok, slot][:, None] * y
    return routed + shared_hidden @ mx.dequantize(*shared[2]).T


def forward_mx(x, router_w, corr_bias,
               experts: Callable[[int], MxExpert],
               shared: MxExpert,
               top_k: int, scale: float,
               force_idx: Optional[np.ndarray] = None,
               routing: Optional[Routing] = None,
               n_group: int = 1, topk_group: int = 1,
               group_topk: int = 2) -> Tuple[np.ndarray, Routing]:
    """The layer with MXFP8 expert weights (``oracle.mx``): ``(out, routing)``.

    Routing (steps 1-4) runs on the input as given, exactly as in ``forward``.
    The expert products take the input quantised to MXFP8 per token along the
    hidden dimension (blocks of 32), and the gated hidden values quantised the
    same way along the expert width; everything else is ``forward``.
    """
    xd = decode(x)
    r = routing if routing is not None else route(xd, router_w, corr_bias, top_k, scale, force_idx,
                                                  n_group, topk_group, group_topk)
    xq = mx.fake_quantize(xd)
    T, D = xd.shape
    routed = np.zeros((T, D))
    for e in np.unique(r.idx):
        tok, slot = np.nonzero(r.idx == e)
        y = expert_mlp_mx(xq[tok], *experts(int(e)))
        routed[tok] += r.weight[tok, slot][:, None] * y
    out = routed + expert_mlp_mx(xq, *shared)
    return out, r
