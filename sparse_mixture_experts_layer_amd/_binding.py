"""ctypes declarations of include/moe_layer.h (argument marshalling only).

The shared library is lib/libmoe_mi355x.so inside this package, built by
`python -m sparse_mixture_experts_layer_amd.build` (with --debug: the
index-checking build in lib/debug/, which the environment variable
MOE_MI355X_LIB can name instead).  There is no fallback: if the library is
missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_mi355x.so")
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "debug",
                              "libmoe_mi355x.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, \
    MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE = range(8)
MOE_F32, MOE_BF16, MOE_INT4_G32 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_BIAS_LOGIT, MOE_BIAS_SELECT = 0, 1
MOE_STAGE_EVENTS = 6
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # scratch of moe_layer_forward_noalloc, per GPU
MOE_ABI_VERSION = 3     # the header these declarations follow
STAGES = ("router", "dispatch", "gate_up", "down", "combine")


class MoeLayerConfig(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("max_tokens", C.c_int32),
                ("score", C.c_int32), ("renormalize", C.c_int32), ("routed_scale", C.c_float),
                ("bias_mode", C.c_int32), ("act_dtype", C.c_int32), ("weight_dtype", C.c_int32),
                ("swiglu_limit", C.c_float), ("swiglu_limit_shared", C.c_float)]


class MoeWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                           "sc_gate", "sc_up", "sc_down", "sc_s_gate", "sc_s_up",
                                           "sc_s_down")]


class MoeRoute(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_idx", "topk_w", "topk_gap", "expert_counts",
                                           "expert_offsets", "perm", "inv", "debug_flag")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_str(status)}: {detail}")
        self.status = status


_lib = None


def load() -> C.CDLL:
    """Loads the library once.  torch is imported first so that the process
    uses a single HIP runtime (the one torch ships)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds libamdhip64 before the library needs it)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"MoE HIP library not built: {LIB_PATH} is missing "
                           "(run: python -m sparse_mixture_experts_layer_amd.build)")
    lib = C.CDLL(LIB_PATH)
    lib.moe_abi_version.restype = C.c_int
    lib.moe_abi_version.argtypes = []
    lib.moe_debug_checks.restype = C.c_int
    lib.moe_debug_checks.argtypes = []
    if lib.moe_abi_version() != MOE_ABI_VERSION:   # struct layouts below would not match
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.moe_abi_version()}, these bindings "
                           f"expect {MOE_ABI_VERSION} (rebuild: python -m "
                           "sparse_mixture_experts_layer_amd.build)")
    lib.moe_layer_create.restype = C.c_int
    lib.moe_layer_create.argtypes = [C.POINTER(MoeLayerConfig), C.c_int, C.POINTER(C.c_void_p)]
    lib.moe_layer_destroy.restype = None
    lib.moe_layer_destroy.argtypes = [C.c_void_p]
    lib.moe_layer_packed_bytes.restype = C.c_size_t
    lib.moe_layer_packed_bytes.argtypes = [C.c_void_p]
    lib.moe_layer_workspace_bytes.restype = C.c_size_t
    lib.moe_layer_workspace_bytes.argtypes = [C.c_void_p, C.c_int32]
    lib.moe_layer_pack_weights.restype = C.c_int
    lib.moe_layer_pack_weights.argtypes = [C.c_void_p, C.POINTER(MoeWeights), C.c_void_p,
                                           C.c_void_p]
    lib.moe_layer_forward.restype = C.c_int
    lib.moe_layer_forward.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                      C.POINTER(MoeRoute), C.c_void_p]
    lib.moe_layer_forward_timed.restype = C.c_int
    lib.moe_layer_forward_timed.argtypes = lib.moe_layer_forward.argtypes + [C.c_void_p]
    lib.moe_layer_forward_noalloc.restype = C.c_int
    lib.moe_layer_forward_noalloc.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                              C.c_void_p, C.c_void_p, C.c_void_p,
                                              C.POINTER(MoeRoute), C.c_void_p]
    lib.moe_status_str.restype = C.c_char_p
    lib.moe_status_str.argtypes = [C.c_int]
    lib.moe_last_error.restype = C.c_char_p
    lib.moe_last_error.argtypes = []
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def last_error() -> str:
    return load().moe_last_error().decode()


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where, last_error())


_hip = None


def memcpy_d2d_async(dst: int, src: int, nbytes: int, stream: int) -> None:
    """hipMemcpyAsync device to device on `stream`, through the HIP runtime the
    process already loaded (torch's)."""
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so.7")
        h.hipMemcpyAsync.restype = C.c_int
        h.hipMemcpyAsync.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
        _hip = h
    HIP_MEMCPY_DEVICE_TO_DEVICE = 3
    if _hip.hipMemcpyAsync(dst, src, nbytes, HIP_MEMCPY_DEVICE_TO_DEVICE, stream) != 0:
        raise RuntimeError("hipMemcpyAsync failed")


# hip_runtime_api.h: an event that skips the system-scope fence of its record
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class StageEvents:
    """Sets of MOE_STAGE_EVENTS HIP events for moe_layer_forward_timed (one set
    per call, so back-to-back calls can be read afterwards), created and read
    through the HIP runtime the process already loaded (torch's).

    The events only time the stages: they are created with
    hipEventDisableSystemFence, so recording one does not write back and
    invalidate the caches (with default events the six records of a decode
    step add ~20 us to it, with these ~10 us).  Waiting on one therefore says
    nothing about the visibility of the layer's outputs; synchronise the
    stream or device before reading them."""

    def __init__(self, sets: int = 1, only=None):
        """only: the stage boundaries to record (indices 0..MOE_STAGE_EVENTS-1),
        all by default; the others stay NULL and are not recorded."""
        load()
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.sets = sets
        self.only = tuple(range(MOE_STAGE_EVENTS)) if only is None else tuple(sorted(only))
        self.array = (C.c_void_p * (MOE_STAGE_EVENTS * sets))()
        for s in range(sets):
            for i in self.only:
                ev = C.c_void_p()
                if self.hip.hipEventCreateWithFlags(C.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                self.array[s * MOE_STAGE_EVENTS + i] = ev

    def ptr(self, s: int = 0) -> int:
        """Address of event set s (a hipEvent_t[MOE_STAGE_EVENTS])."""
        return C.addressof(self.array) + s * MOE_STAGE_EVENTS * C.sizeof(C.c_void_p)

    def elapsed_ms(self, s: int, a: int, b: int) -> float:
        """Time (ms) from boundary a to boundary b of set s (synchronises)."""
        base = s * MOE_STAGE_EVENTS
        self.hip.hipEventSynchronize(self.array[base + b])
        ms = C.c_float()
        if self.hip.hipEventElapsedTime(C.byref(ms), self.array[base + a],
                                        self.array[base + b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def stage_ms(self, s: int = 0):
        """Durations (ms) of the 5 stages recorded in set s (synchronises);
        None for a stage whose boundaries were not both recorded."""
        return [self.elapsed_ms(s, i, i + 1) if i in self.only and i + 1 in self.only else None
                for i in range(MOE_STAGE_EVENTS - 1)]

    def __del__(self):
        try:
            for i in range(MOE_STAGE_EVENTS * self.sets):
                if self.array[i]:
                    self.hip.hipEventDestroy(self.array[i])
        except Exception:
            pass
