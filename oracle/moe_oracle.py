"""Oracle for the sparse MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow CPU implementation (NumPy, float64) of what the layer computes,
used only by tests/, by __graft_entry__.smoke() and by the benchmark's CPU
baseline leg.  The GPU library never imports, calls or links anything here,
and nothing here imports the GPU library.

What the layer computes (sources: the five pages about Step-3.5-Flash):

* A sparse mixture of experts FFN: many experts are stored, only a few run per
  token (q4km.ai "Step-3.5-Flash", "Technical Overview" and "Architecture
  highlights"; nipponese.news article, architecture section).
* 288 routed experts, top-8 routing (llm-atlas "Step-3.5-Flash", section
  "FFN / MoE"; config fields moe_num_experts, moe_top_k).
* Expert width 1280 and an always-on shared expert of width 1280 (config fields
  moe_intermediate_size, share_expert_dim).
* Renormalised expert weights (config field norm_expert_weight: true; the
  Step-3 comparison table shows it was false for Step-3).
* Router computed in fp32 (config field need_fp32_gate: true) with a per-expert
  router bias (use_moe_router_bias: true).

Readings taken where the pages are silent or disagree (each is listed in the
design notes):

* Scoring: softmax over all experts.  The config lists
  moe_router_activation = sigmoid with moe_router_scaling_factor = 3; that
  variant is provided too (score="sigmoid"), the softmax form is the default.
* Tie rule: experts are ordered by descending fp32 logit, equal logits by
  ascending expert index.
* Expert FFN: SiLU-gated (gate -> SiLU, up -> linear, h = silu(gate) * up,
  y = down h).  Three matrices per expert are implied by the 196B total
  parameter count; gating is implied by the swiglu_limits fields, whose value
  is 0 (no clamp) for every MoE layer.  A nonzero limit L (7 for the routed
  and 16 for the shared experts of the last layers) is read as clamping the
  gate projection to at most L and the up projection to [-L, L].  The pages
  give the limit values only, so this clamp is parity unpinned: its pin checks
  the reading by hand, nothing on the pages checks the reading.
* No bias terms in the expert linears; the shared expert is added unweighted.
* Router bias: added to the logits before selection and weighting
  (bias_mode="logit"); bias_mode="select" uses it for selection only.

Precision: the router logits are accumulated in float64 and rounded once to
float32, because the pages fix the gate precision at fp32 and the selection is
an integer decision taken on fp32 values.  Everything else is float64.

Parity pins (tests/test_oracle_pins.py): brute-force full-sort top-k, the
closed-form renormalised weights, k = 1 and k = E special cases, identical
experts reducing to a dense SwiGLU FFN, a hand-computed two-expert case
(tests/golden/hand_two_expert.json), expert-relabelling and token-independence
invariants, INT4 dequantisation bounds, dispatch against a Python sort, and
hand-evaluated SwiGLU limits.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Tuple

import numpy as np

Expert = Tuple[np.ndarray, np.ndarray, np.ndarray]  # (W_gate [I][H], W_up [I][H], W_down [H][I])


# --------------------------------------------------------------------------- router

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None,
                  bias_in_logits: bool = True) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e]), accumulated in float64 and
    rounded once to float32 (need_fp32_gate; use_moe_router_bias)."""
    l64 = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None and bias_in_logits:
        l64 = l64 + np.asarray(bias, np.float64)[None, :]
    return l64.astype(np.float32)


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """k rounds of arg-max per row: the largest remaining score wins, and among
    equal scores the lowest expert index (np.argmax returns the first)."""
    scores = np.array(scores, dtype=np.float64, copy=True)
    t, e = scores.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= number of experts")
    idx = np.empty((t, k), dtype=np.int64)
    for j in range(k):
        best = np.argmax(scores, axis=1)
        idx[:, j] = best
        scores[np.arange(t), best] = -np.inf
    return idx


def gate_weights(logits32: np.ndarray, idx: np.ndarray, score: str = "softmax",
                 renormalize: bool = True, routed_scale: float = 1.0) -> np.ndarray:
    """Weights of the selected experts, in float64, from the fp32 logits.

    softmax: p = exp(l - max l) / sum over all experts; sigmoid: p = 1/(1+exp(-l)).
    With renormalisation (norm_expert_weight) w_j = p_sel_j / sum_i p_sel_i,
    else w_j = p_sel_j; then w *= routed_scale."""
    l = np.asarray(logits32, np.float64)
    if score == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        p = 1.0 / (1.0 + np.exp(-l))
    else:
        raise ValueError(score)
    sel = np.take_along_axis(p, idx, axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel * routed_scale


def route(x, w_router, bias, top_k, score="softmax", renormalize=True, routed_scale=1.0,
          bias_mode="logit"):
    """Returns (idx [T][k] int64, w [T][k] float64, logits [T][E] float32).

    bias_mode "logit": bias enters the logits used for selection and weights.
    bias_mode "select": bias only shifts the selection scores; weights use the
    unbiased logits."""
    if bias_mode not in ("logit", "select"):
        raise ValueError(bias_mode)
    l32 = router_logits(x, w_router, bias, bias_in_logits=(bias_mode == "logit"))
    sel_scores = l32
    if bias is not None and bias_mode == "select":
        sel_scores = (l32.astype(np.float64) + np.asarray(bias, np.float64)[None, :]).astype(np.float32)
    idx = select_topk(sel_scores, top_k)
    w = gate_weights(l32, idx, score, renormalize, routed_scale)
    return idx, w, l32


def topk_gap(scores32: np.ndarray, k: int) -> np.ndarray:
    """Per token, (k-th largest - (k+1)-th largest) selection score; +inf when
    k equals the number of experts.  Tokens with a gap below the near-tie band
    may legitimately be routed differently by a different summation order."""
    s = np.sort(np.asarray(scores32, np.float64), axis=1)[:, ::-1]
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# --------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
               w_down: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """y = W_down (silu(g) * u), g = W_gate x, u = W_up x, for each row of x_rows
    (float64).

    limit > 0 bounds the two projections before the product: g to at most
    limit, u to [-limit, limit].  Source: llm-atlas "Step-3.5-Flash", config
    fields swiglu_limits (0 on every layer but the last two, 7 there) and
    swiglu_limits_shared (16 on the last layer, for the shared expert).  The
    pages give only the values; this clamp form is the reading taken."""
    x_rows = np.asarray(x_rows, np.float64)
    g = x_rows @ np.asarray(w_gate, np.float64).T
    u = x_rows @ np.asarray(w_up, np.float64).T
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return (silu(g) * u) @ np.asarray(w_down, np.float64).T


def dequant_int4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """INT4 group-32 weights -> float64: w[n, k] = s[n, k // 32] * (u[n, k] - 8),
    u the nibble of element k (byte k // 2, low nibble for even k).  Exact."""
    packed = np.asarray(packed, np.uint8)
    lo = (packed & 0xF).astype(np.int64) - 8
    hi = (packed >> 4).astype(np.int64) - 8
    q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    s = np.asarray(scales, np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(s, 32, axis=-1)


# --------------------------------------------------------------------------- layer

def forward(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
            experts: Callable[[int], Expert], shared: Optional[Expert], top_k: int,
            score: str = "softmax", renormalize: bool = True, routed_scale: float = 1.0,
            bias_mode: str = "logit", force_idx: Optional[np.ndarray] = None,
            swiglu_limit: float = 0.0, swiglu_limit_shared: float = 0.0):
    """The whole layer on the host.  Returns (y [T][H] float64, idx, w, logits32).

    experts(e) returns that expert's (W_gate, W_up, W_down); it is called once
    per expert that at least one token selected, so large layers can be
    materialised one expert at a time.  force_idx, if given, replaces the
    selection (the weights are still computed from the logits).
    swiglu_limit / swiglu_limit_shared: the routed / shared experts' SwiGLU
    limits (0 = none; see swiglu_ffn)."""
    x = np.asarray(x, np.float64)
    t = x.shape[0]
    idx, w, l32 = route(x, w_router, bias, top_k, score, renormalize, routed_scale, bias_mode)
    if force_idx is not None:
        idx = np.asarray(force_idx, np.int64)
        w = gate_weights(l32, idx, score, renormalize, routed_scale)
    y = np.zeros((t, x.shape[1]), np.float64)
    if shared is not None:
        y += swiglu_ffn(x, *shared, limit=swiglu_limit_shared)
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        y_e = swiglu_ffn(x[tok], *experts(int(e)), limit=swiglu_limit)
        y[tok] += w[tok, slot][:, None] * y_e
    return y, idx, w, l32


def dispatch(idx: np.ndarray, num_experts: int):
    """Reference expert dispatch for pair ids p = t*k + j.

    counts[e]: number of pairs routed to e; offsets: exclusive prefix sum with
    offsets[E] = number of pairs; perm[r]: the pair id stored at permuted row r,
    rows grouped by expert and ordered by token inside a group; inv[p]: the row
    of pair p."""
    idx = np.asarray(idx, np.int64)
    t, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.empty(t * k, np.int64)
    fill = offsets[:-1].copy()
    for p in range(t * k):            # pairs visited in token order: a stable counting sort
        e = flat[p]
        perm[fill[e]] = p
        fill[e] += 1
    inv = np.empty(t * k, np.int64)
    inv[perm] = np.arange(t * k)
    return counts, offsets, perm, inv
