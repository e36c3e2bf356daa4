"""The C-ABI library loads and exports every declared symbol; argument
validation answers on a host without a GPU (no compute calls)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_mixture_experts_layer_amd import _binding
    return _binding.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "moe_layer_forward" in names and "moe_layer_create" in names
    for n in names:
        assert hasattr(lib, n), f"library does not export {n}"


def test_abi_version(lib):
    """The header's version, the library's and the bindings' agree (the
    bindings refuse a library of another version: its structs differ)."""
    from sparse_mixture_experts_layer_amd import _binding as B
    m = re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.moe_abi_version() == int(m.group(1)) == B.MOE_ABI_VERSION == 3


def _cfg(**kw):
    from sparse_mixture_experts_layer_amd import _binding as B
    base = dict(hidden=256, num_experts=16, top_k=2, inter=64, shared_inter=64, max_tokens=64,
                score=0, renormalize=1, routed_scale=1.0, bias_mode=0, act_dtype=B.MOE_BF16,
                weight_dtype=B.MOE_BF16)
    base.update(kw)
    return B.MoeLayerConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), 2), (dict(top_k=17), 2), (dict(top_k=17, num_experts=16), 2),
    (dict(num_experts=513), 2), (dict(hidden=100), 2), (dict(inter=48), 2),
    (dict(shared_inter=-32), 2), (dict(max_tokens=0), 2), (dict(act_dtype=2), 3),
    (dict(weight_dtype=0), 3), (dict(score=5), 3), (dict(bias_mode=2), 3),
    (dict(routed_scale=0.0), 2), (dict(weight_dtype=2, inter=64), 2),
    (dict(swiglu_limit=-1.0), 2), (dict(swiglu_limit_shared=float("inf")), 2),
    (dict(swiglu_limit=float("nan")), 2),
])
def test_config_validation(lib, kw, status):
    from sparse_mixture_experts_layer_amd import _binding as B
    h = C.c_void_p()
    st = lib.moe_layer_create(C.byref(_cfg(**kw)), 0, C.byref(h))
    assert st == status, (st, B.last_error())
    assert B.last_error()
    assert not h.value


def test_null_arguments(lib):
    from sparse_mixture_experts_layer_amd import _binding as B
    assert lib.moe_layer_create(None, 0, None) == B.MOE_ERR_NULL
    h = C.c_void_p()
    assert lib.moe_layer_create(None, 0, C.byref(h)) == B.MOE_ERR_NULL
    assert lib.moe_layer_forward(None, 1, None, None, None, None, None, None, 0, None,
                                 None) == B.MOE_ERR_NULL
    assert lib.moe_layer_packed_bytes(None) == 0
    lib.moe_layer_destroy(None)
    assert lib.moe_status_str(B.MOE_ERR_WORKSPACE) == b"MOE_ERR_WORKSPACE"


def test_no_device_reported(lib):
    """On a host without a GPU a valid config fails with MOE_ERR_DEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from sparse_mixture_experts_layer_amd import _binding as B
    h = C.c_void_p()
    assert lib.moe_layer_create(C.byref(_cfg()), 0, C.byref(h)) == B.MOE_ERR_DEVICE


def test_debug_build_exports_the_same_symbols(lib):
    """The index-checking build (build --debug) exports the same entry points
    and says so; the release build says it has no checks."""
    from sparse_mixture_experts_layer_amd import _binding as B
    assert os.path.exists(B.DEBUG_LIB_PATH), "debug library not built"
    dbg = C.CDLL(B.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(dbg, n), f"debug library does not export {n}"
    dbg.moe_debug_checks.restype = C.c_int
    assert dbg.moe_debug_checks() == 1
    if os.path.realpath(B.LIB_PATH) != os.path.realpath(B.DEBUG_LIB_PATH):
        assert lib.moe_debug_checks() == 0
