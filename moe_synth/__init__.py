"""Seeded synthetic inputs for the sparse MoE FFN layer (Step-3.5-Flash shape).

This module is the only code shared by the oracle tests and the GPU path: it
draws tensors and nothing else.  It holds none of the layer's arithmetic
(no routing, no expert math).  The one transformation it applies besides
drawing is the offline INT4 weight quantiser, because quantised weights are an
*input* of the INT4 path (the layer itself only ever dequantises).

Shapes come from the llm-atlas model card "Step-3.5-Flash", tables "Faits cles"
and "Champs bruts du config.json" (hidden_size 4096, moe_num_experts 288,
moe_top_k 8, moe_intermediate_size 1280, share_expert_dim 1280, torch_dtype
bfloat16).  Value distributions: activations N(0,1); weights N(0, 1/fan_in),
fan_in = hidden for gate/up/router and = the intermediate width for down,
rounded to bf16 (round to nearest even).

Every tensor (and every expert's slice of it) has its own seed, derived from
(seed, workload index, tensor id, expert) with numpy's SeedSequence, so any
expert can be regenerated alone.  Generation runs through torch's generator on
the requested device (CPU or GPU); for one device and one torch build the
values are reproducible.  Tensors drawn on the GPU are copied to the host for
the oracle: they are inputs, produced by torch's RNG, not by the layer.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))


@dataclass(frozen=True)
class LayerShape:
    name: str
    tokens: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    shared_inter: int
    act_dtype: str = "bf16"        # "bf16" | "f32"
    weight_dtype: str = "bf16"     # "bf16" | "int4_g32"
    routing: str = "uniform"       # "uniform" (no bias) | "zipf" (Zipf-calibrated bias) |
                                   # "bias" (seeded N(0, 0.1^2) per-expert bias)
    renormalize: bool = True
    index: int = 0                 # workload index, part of every seed
    x_scale: float = 1.0           # activations drawn from N(0, x_scale^2)
    swiglu_limit: float = 0.0      # routed experts' SwiGLU limit (0 = none)
    swiglu_limit_shared: float = 0.0  # shared expert's SwiGLU limit (0 = none)
    score: str = "softmax"         # router scores: "softmax" | "sigmoid"
    routed_scale: float = 1.0      # factor on the routed weights
    bias_mode: str = "logit"       # router bias in the logits ("logit") or the selection only

    @property
    def pairs(self) -> int:
        return self.tokens * self.top_k

    def with_tokens(self, tokens: int) -> "LayerShape":
        return LayerShape(**{**self.__dict__, "tokens": tokens})

    def replace(self, **kw) -> "LayerShape":
        return LayerShape(**{**self.__dict__, **kw})


STEP35 = dict(hidden=4096, experts=288, top_k=8, inter=1280, shared_inter=1280)
# Step-3's MoE layer (llm-atlas "Step-3.5-Flash", table comparing it with
# Step-3): hidden 7168, 48 experts, top-3, width 5120, no renormalisation
STEP3 = dict(hidden=7168, experts=48, top_k=3, inter=5120, shared_inter=5120, renormalize=False)
# the dense SwiGLU FFN of the first layers (intermediate_size 11264) as one expert
DENSE = dict(hidden=4096, experts=1, top_k=1, inter=11264, shared_inter=0)

# The workloads.  Index 0 is the tiny case the oracle finishes in
# milliseconds; 1 is single-stream-batch decode; 2 is a multi-token-prediction
# verify batch (64 streams x (1+3) tokens) with Zipf expert popularity; 3 is a
# prefill chunk; 4 is decode with INT4 group-32 weights; 5 is decode through
# one of the last layers, whose SwiGLU limits are 7 (routed) and 16 (shared)
# (llm-atlas "Step-3.5-Flash", config fields swiglu_limits and
# swiglu_limits_shared), with activations drawn 8x wider so that the clamps
# act: the projections then have a standard deviation near 8, and about a
# third of the routed up values and a twentieth of the shared ones lie beyond
# their limit.  6 is decode under the page's router configuration (sigmoid
# scores, a per-expert router bias -- drawn N(0, 0.1^2) here, the pages give
# no values -- and routed weights scaled by 3; llm-atlas config fields
# moe_router_activation, use_moe_router_bias, moe_router_scaling_factor);
# 7 and 8 are Step-3's MoE shape at a decode batch and a 4096-token chunk
# (256 rows per expert); 9 and 10 are the dense FFN as one expert at a
# decode batch and a 16384-token chunk.
WORKLOADS = {
    "tiny": LayerShape("tiny", 64, 256, 16, 2, 64, 64, act_dtype="f32", index=0),
    "decode": LayerShape("decode", 32, **STEP35, index=1),
    "verify": LayerShape("verify", 256, **STEP35, routing="zipf", index=2),
    "prefill": LayerShape("prefill", 16384, **STEP35, index=3),
    "int4_decode": LayerShape("int4_decode", 32, **STEP35, weight_dtype="int4_g32", index=4),
    "mtp_decode": LayerShape("mtp_decode", 32, **STEP35, x_scale=8.0, swiglu_limit=7.0,
                             swiglu_limit_shared=16.0, index=5),
    "page_router_decode": LayerShape("page_router_decode", 32, **STEP35, routing="bias",
                                     score="sigmoid", routed_scale=3.0, index=6),
    "step3_decode": LayerShape("step3_decode", 32, **STEP3, index=7),
    "step3_prefill": LayerShape("step3_prefill", 4096, **STEP3, index=8),
    "dense_decode": LayerShape("dense_decode", 32, **DENSE, index=9),
    "dense_prefill": LayerShape("dense_prefill", 16384, **DENSE, index=10),
}

# tensor ids (part of the seed)
T_X, T_ROUTER, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN, T_BIAS = range(9)


def seed_for(seed: int, workload: int, tensor: int, expert: int = 0) -> int:
    ss = np.random.SeedSequence([seed, workload, tensor, expert])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, scale: float, device, s: int, dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, s), device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)


def zipf_bias(num_experts: int) -> np.ndarray:
    """Per-expert logit bias (fp32) giving capped Zipf(s=1) popularity.

    Calibrated offline by calibrate_zipf_bias.py for 288 experts, top-8."""
    if num_experts != 288:
        raise ValueError("the Zipf bias is calibrated for 288 experts only")
    return np.load(os.path.join(_HERE, "zipf_bias_e288.npy"))


def quantize_int4_g32(w: torch.Tensor):
    """Symmetric INT4 with one fp16 scale per 32 consecutive input channels.

    w: [..., N, K] float tensor, K % 32 == 0.  Per group: s = fp16(absmax / 7);
    q = clamp(round_half_even(w / s), -8, 7) using the fp16-rounded s; s == 0
    gives q = 0.  Returns (packed, scales): packed uint8 [..., N, K/2] holding
    u = q + 8 with element k in byte k/2, low nibble for even k; scales fp16
    [..., N, K/32]."""
    *lead, n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    g = w.float().reshape(*lead, n, k // 32, 32)
    s = (g.abs().amax(dim=-1) / 7.0).to(torch.float16)
    sf = s.float().unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(g / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(g))
    q = q.clamp_(-8, 7).to(torch.int16).reshape(*lead, n, k)
    u = (q + 8).to(torch.uint8)
    packed = (u[..., 0::2] | (u[..., 1::2] << 4)).contiguous()
    return packed, s.contiguous()


def unpack_int4(packed: torch.Tensor) -> torch.Tensor:
    """Inverse of the nibble packing: uint8 [..., K/2] -> int8 q [..., K]."""
    lo = (packed & 0xF).to(torch.int8) - 8
    hi = (packed >> 4).to(torch.int8) - 8
    return torch.stack([lo, hi], dim=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


@dataclass
class LayerInputs:
    shape: LayerShape
    x: torch.Tensor                      # [T][H] f32 or bf16
    router_w: torch.Tensor               # [E][H] bf16
    router_bias: Optional[torch.Tensor]  # [E] f32 or None
    w_gate: Optional[torch.Tensor] = None  # [E][I][H] bf16   (bf16 weights)
    w_up: Optional[torch.Tensor] = None    # [E][I][H] bf16
    w_down: Optional[torch.Tensor] = None  # [E][H][I] bf16
    s_gate: Optional[torch.Tensor] = None  # [Is][H] bf16
    s_up: Optional[torch.Tensor] = None    # [Is][H] bf16
    s_down: Optional[torch.Tensor] = None  # [H][Is] bf16
    # INT4 weights: name -> (packed uint8 [.., N, K/2], scales fp16 [.., N, K/32])
    q: dict = field(default_factory=dict)

    @property
    def device(self):
        return self.x.device


def make_layer(shape: LayerShape, seed: int = 0, device="cpu",
               tokens: Optional[int] = None) -> LayerInputs:
    """Draw every input of one layer call on `device`.

    tokens overrides shape.tokens (the activations' seed does not depend on
    the token count; rows are drawn in one piece so a prefix of a larger draw
    is *not* implied)."""
    dev = torch.device(device)
    wl = shape.index
    T = shape.tokens if tokens is None else tokens
    H, E, I, Is = shape.hidden, shape.experts, shape.inter, shape.shared_inter
    act = torch.float32 if shape.act_dtype == "f32" else torch.bfloat16
    x = _normal((T, H), shape.x_scale, dev, seed_for(seed, wl, T_X), act)
    router_w = _normal((E, H), 1.0 / math.sqrt(H), dev, seed_for(seed, wl, T_ROUTER), torch.bfloat16)
    bias = None
    if shape.routing == "zipf":
        bias = torch.from_numpy(zipf_bias(E)).to(dev)
    elif shape.routing == "bias":
        bias = _normal((E,), 0.1, dev, seed_for(seed, wl, T_BIAS), torch.float32)
    out = LayerInputs(shape, x, router_w, bias)

    def stacked(tensor_id, n, k, fan_in):
        w = torch.empty((E, n, k), dtype=torch.bfloat16, device=dev)
        for e in range(E):
            w[e] = _normal((n, k), 1.0 / math.sqrt(fan_in), dev, seed_for(seed, wl, tensor_id, e),
                           torch.bfloat16)
        return w

    w_gate = stacked(T_GATE, I, H, H)
    w_up = stacked(T_UP, I, H, H)
    w_down = stacked(T_DOWN, H, I, I)
    s_gate = s_up = s_down = None
    if Is > 0:
        s_gate = _normal((Is, H), 1.0 / math.sqrt(H), dev, seed_for(seed, wl, T_SGATE), torch.bfloat16)
        s_up = _normal((Is, H), 1.0 / math.sqrt(H), dev, seed_for(seed, wl, T_SUP), torch.bfloat16)
        s_down = _normal((H, Is), 1.0 / math.sqrt(Is), dev, seed_for(seed, wl, T_SDOWN), torch.bfloat16)
    if shape.weight_dtype == "int4_g32":
        for name, w in (("gate", w_gate), ("up", w_up), ("down", w_down),
                        ("s_gate", s_gate), ("s_up", s_up), ("s_down", s_down)):
            if w is not None:
                out.q[name] = quantize_int4_g32(w)
        del w_gate, w_up, w_down
    else:
        out.w_gate, out.w_up, out.w_down = w_gate, w_up, w_down
        out.s_gate, out.s_up, out.s_down = s_gate, s_up, s_down
    return out


def host_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact float64 host copy of a float tensor (bf16/f16/f32 widen exactly;
    widened on the tensor's own device, then copied)."""
    if t is None:
        return None
    return t.detach().to(torch.float64).to("cpu").numpy()
