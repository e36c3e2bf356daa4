"""MoELayer: a thin Python wrapper over the C ABI in include/moe_layer.h.

torch provides device memory (the packed weights, workspace and outputs are
torch tensors) and the stream (the current torch stream); every step of the
layer runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B

_SCORES = {"softmax": B.MOE_SCORE_SOFTMAX, "sigmoid": B.MOE_SCORE_SIGMOID}
_BIAS = {"logit": B.MOE_BIAS_LOGIT, "select": B.MOE_BIAS_SELECT}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _need_bytes(t: torch.Tensor, name: str, min_bytes: int, device) -> None:
    """A device byte buffer: contiguous uint8 of at least min_bytes."""
    if t.dtype != torch.uint8 or t.dim() != 1 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 1-D torch.uint8 tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.numel() < min_bytes:
        raise ValueError(f"{name} has {t.numel()} bytes, {min_bytes} needed")


@dataclass
class Route:
    """Routing results of one forward (views into the workspace)."""
    topk_idx: torch.Tensor       # [T][k] int32
    topk_w: torch.Tensor         # [T][k] float32
    topk_gap: torch.Tensor       # [T] float32
    expert_counts: torch.Tensor  # [E] int32
    expert_offsets: torch.Tensor  # [E+1] int32
    perm: torch.Tensor           # [T*k] int32
    inv: torch.Tensor            # [T*k] int32
    debug_flag: Optional[torch.Tensor] = None  # [2] int32 (index-checking builds only)


class MoELayer:
    def __init__(self, hidden: int, num_experts: int, top_k: int, inter: int, shared_inter: int,
                 max_tokens: int, score: str = "softmax", renormalize: bool = True,
                 routed_scale: float = 1.0, bias_mode: str = "logit",
                 act_dtype: torch.dtype = torch.bfloat16, weight_dtype: str = "bf16",
                 swiglu_limit: float = 0.0, swiglu_limit_shared: float = 0.0,
                 device: int = 0):
        self.lib = B.load()
        self.cfg = B.MoeLayerConfig(
            hidden=hidden, num_experts=num_experts, top_k=top_k, inter=inter,
            shared_inter=shared_inter, max_tokens=max_tokens, score=_SCORES[score],
            renormalize=int(bool(renormalize)), routed_scale=float(routed_scale),
            bias_mode=_BIAS[bias_mode],
            act_dtype=B.MOE_F32 if act_dtype == torch.float32 else B.MOE_BF16,
            weight_dtype=B.MOE_INT4_G32 if weight_dtype == "int4_g32" else B.MOE_BF16,
            swiglu_limit=float(swiglu_limit), swiglu_limit_shared=float(swiglu_limit_shared))
        if act_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("act_dtype must be torch.float32 or torch.bfloat16")
        self.act_dtype = act_dtype
        self.weight_dtype = weight_dtype
        self.device = torch.device("cuda", device)
        h = C.c_void_p()
        B.check(self.lib.moe_layer_create(C.byref(self.cfg), device, C.byref(h)),
                "moe_layer_create")
        self._h = h
        self.packed: Optional[torch.Tensor] = None

    @classmethod
    def from_shape(cls, shape, max_tokens: Optional[int] = None, device: int = 0, **kw):
        """Builds a layer from a moe_synth.LayerShape-like object."""
        return cls(shape.hidden, shape.experts, shape.top_k, shape.inter, shape.shared_inter,
                   max_tokens or shape.tokens, renormalize=shape.renormalize,
                   act_dtype=torch.float32 if shape.act_dtype == "f32" else torch.bfloat16,
                   weight_dtype=shape.weight_dtype, device=device,
                   **{"swiglu_limit": getattr(shape, "swiglu_limit", 0.0),
                      "swiglu_limit_shared": getattr(shape, "swiglu_limit_shared", 0.0),
                      "score": getattr(shape, "score", "softmax"),
                      "routed_scale": getattr(shape, "routed_scale", 1.0),
                      "bias_mode": getattr(shape, "bias_mode", "logit"), **kw})

    def close(self) -> None:
        if getattr(self, "_h", None):
            self.lib.moe_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ sizes
    @property
    def packed_bytes(self) -> int:
        return int(self.lib.moe_layer_packed_bytes(self._h))

    def workspace_bytes(self, num_tokens: int) -> int:
        return int(self.lib.moe_layer_workspace_bytes(self._h, num_tokens))

    def _stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    # ------------------------------------------------------------------ weights
    def pack(self, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
             scales: Optional[dict] = None) -> torch.Tensor:
        """Packs canonical weights (see moe_weights_t) into a new device buffer.

        bf16: w_* bf16 [E][I][H] / [E][H][I]; s_* bf16 [Is][H] / [H][Is].
        int4_g32: w_* / s_* uint8 nibble tensors of the same element order with
        K/2 bytes per row, and scales = {"gate", "up", "down", "s_gate", "s_up",
        "s_down"} -> fp16 [..][N][K/32]."""
        c = self.cfg
        E, H, I, Is = c.num_experts, c.hidden, c.inter, c.shared_inter
        int4 = self.weight_dtype == "int4_g32"
        wdt = torch.uint8 if int4 else torch.bfloat16
        kdiv = 2 if int4 else 1
        dev = self.device
        _need(w_gate, "w_gate", wdt, (E, I, H // kdiv), dev)
        _need(w_up, "w_up", wdt, (E, I, H // kdiv), dev)
        _need(w_down, "w_down", wdt, (E, H, I // kdiv), dev)
        if Is:
            _need(s_gate, "s_gate", wdt, (Is, H // kdiv), dev)
            _need(s_up, "s_up", wdt, (Is, H // kdiv), dev)
            _need(s_down, "s_down", wdt, (H, Is // kdiv), dev)
        w = B.MoeWeights(w_gate=_ptr(w_gate), w_up=_ptr(w_up), w_down=_ptr(w_down),
                         s_gate=_ptr(s_gate) if Is else None, s_up=_ptr(s_up) if Is else None,
                         s_down=_ptr(s_down) if Is else None)
        if int4:
            if scales is None:
                raise ValueError("INT4 weights need their fp16 scales")
            shapes = {"gate": (E, I, H // 32), "up": (E, I, H // 32), "down": (E, H, I // 32),
                      "s_gate": (Is, H // 32), "s_up": (Is, H // 32), "s_down": (H, Is // 32)}
            for n, shp in shapes.items():
                if n.startswith("s_") and not Is:
                    continue
                _need(scales[n], f"scales[{n}]", torch.float16, shp, dev)
            w.sc_gate, w.sc_up, w.sc_down = (_ptr(scales[n]) for n in ("gate", "up", "down"))
            if Is:
                w.sc_s_gate, w.sc_s_up, w.sc_s_down = (_ptr(scales[n])
                                                       for n in ("s_gate", "s_up", "s_down"))
        packed = torch.empty(self.packed_bytes, dtype=torch.uint8, device=dev)
        B.check(self.lib.moe_layer_pack_weights(self._h, C.byref(w), packed.data_ptr(),
                                                self._stream()), "moe_layer_pack_weights")
        self.packed = packed
        return packed

    def pack_inputs(self, inp) -> torch.Tensor:
        """Packs the weights of a moe_synth.LayerInputs."""
        if self.weight_dtype == "int4_g32":
            q = inp.q
            sc = {n: q[n][1] for n in q}
            return self.pack(q["gate"][0], q["up"][0], q["down"][0], q.get("s_gate", (None,))[0],
                             q.get("s_up", (None,))[0], q.get("s_down", (None,))[0], scales=sc)
        return self.pack(inp.w_gate, inp.w_up, inp.w_down, inp.s_gate, inp.s_up, inp.s_down)

    # ------------------------------------------------------------------ forward
    def forward(self, x: torch.Tensor, router_w: torch.Tensor,
                router_bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None,
                return_route: bool = False, stage_events: Optional["B.StageEvents"] = None,
                event_set: int = 0):
        """y = layer(x).  With stage_events (a _binding.StageEvents) the call goes
        through moe_layer_forward_timed and records event set `event_set`."""
        c = self.cfg
        T = x.shape[0]
        dev = self.device
        _need(x, "x", self.act_dtype, (T, c.hidden), dev)
        _need(router_w, "router_w", torch.bfloat16, (c.num_experts, c.hidden), dev)
        if router_bias is not None:
            _need(router_bias, "router_bias", torch.float32, (c.num_experts,), dev)
        packed = self.packed if packed is None else packed
        if packed is None:
            raise RuntimeError("weights are not packed (call pack first)")
        _need_bytes(packed, "packed", self.packed_bytes, dev)
        if out is None:
            out = torch.empty((T, c.hidden), dtype=self.act_dtype, device=dev)
        else:
            _need(out, "out", self.act_dtype, (T, c.hidden), dev)
        if workspace is None:
            workspace = torch.empty(max(self.workspace_bytes(T), 1), dtype=torch.uint8, device=dev)
        else:   # its size is checked by the library against the batch's plan
            _need_bytes(workspace, "workspace", 0, dev)
        route = B.MoeRoute()
        args = (self._h, T, x.data_ptr(), router_w.data_ptr(), _ptr(router_bias),
                packed.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                C.byref(route), self._stream())
        if stage_events is None:
            B.check(self.lib.moe_layer_forward(*args), "moe_layer_forward")
        else:
            B.check(self.lib.moe_layer_forward_timed(*args, stage_events.ptr(event_set)),
                    "moe_layer_forward_timed")
        if not return_route:
            return out
        return out, self._route_views(route, workspace, T)

    def forward_noalloc(self, x: torch.Tensor, router_w: torch.Tensor,
                        router_bias: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None,
                        return_route: bool = False):
        """y = layer(x) through moe_layer_forward_noalloc: the library's static
        per-GPU scratch replaces the workspace (calls that overlap on one GPU
        race).  With return_route, the routing results are copied out of that
        scratch into new tensors on the current stream."""
        c = self.cfg
        T = x.shape[0]
        dev = self.device
        _need(x, "x", self.act_dtype, (T, c.hidden), dev)
        _need(router_w, "router_w", torch.bfloat16, (c.num_experts, c.hidden), dev)
        if router_bias is not None:
            _need(router_bias, "router_bias", torch.float32, (c.num_experts,), dev)
        packed = self.packed if packed is None else packed
        if packed is None:
            raise RuntimeError("weights are not packed (call pack first)")
        _need_bytes(packed, "packed", self.packed_bytes, dev)
        if out is None:
            out = torch.empty((T, c.hidden), dtype=self.act_dtype, device=dev)
        else:
            _need(out, "out", self.act_dtype, (T, c.hidden), dev)
        route = B.MoeRoute()
        B.check(self.lib.moe_layer_forward_noalloc(
            self._h, T, x.data_ptr(), router_w.data_ptr(), _ptr(router_bias), packed.data_ptr(),
            out.data_ptr(), C.byref(route), self._stream()), "moe_layer_forward_noalloc")
        if not return_route:
            return out
        k, E = c.top_k, c.num_experts

        def copy(ptr, shape, dtype):
            t = torch.empty(shape, dtype=dtype, device=dev)
            if t.numel():
                B.memcpy_d2d_async(t.data_ptr(), ptr, t.numel() * t.element_size(),
                                   self._stream())
            return t

        return out, Route(copy(route.topk_idx, (T, k), torch.int32),
                          copy(route.topk_w, (T, k), torch.float32),
                          copy(route.topk_gap, (T,), torch.float32),
                          copy(route.expert_counts, (E,), torch.int32),
                          copy(route.expert_offsets, (E + 1,), torch.int32),
                          copy(route.perm, (T * k,), torch.int32),
                          copy(route.inv, (T * k,), torch.int32),
                          copy(route.debug_flag, (2,), torch.int32) if route.debug_flag else None)

    def _route_views(self, r: "B.MoeRoute", ws: torch.Tensor, T: int) -> Route:
        c = self.cfg
        base = ws.data_ptr()

        def view(ptr, n, dtype):
            off = ptr - base
            return ws[off:off + n * 4].view(dtype)

        k, E = c.top_k, c.num_experts
        return Route(view(r.topk_idx, T * k, torch.int32).view(T, k),
                     view(r.topk_w, T * k, torch.float32).view(T, k),
                     view(r.topk_gap, T, torch.float32),
                     view(r.expert_counts, E, torch.int32),
                     view(r.expert_offsets, E + 1, torch.int32),
                     view(r.perm, T * k, torch.int32),
                     view(r.inv, T * k, torch.int32),
                     view(r.debug_flag, 2, torch.int32) if r.debug_flag else None)

    __call__ = forward
