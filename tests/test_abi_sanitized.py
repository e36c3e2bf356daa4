"""The host side of the C ABI (csrc/moe_abi.cpp: configuration checks, the
launch plan, argument validation, error reporting) built with AddressSanitizer
and UndefinedBehaviorSanitizer -- host code only, the kernels are the release
objects -- and driven by a C program through every argument-validation path
that answers without a GPU.  Any sanitizer report fails the run."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_mixture_experts_layer_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SAN = ["address", "undefined"]

DRIVER = r"""
#include "moe_layer.h"
#include <math.h>
#include <stdio.h>
#include <string.h>
static moe_layer_config_t base(void) {
  moe_layer_config_t c;
  memset(&c, 0, sizeof c);
  c.hidden = 256; c.num_experts = 16; c.top_k = 2; c.inter = 64; c.shared_inter = 64;
  c.max_tokens = 64; c.score = MOE_SCORE_SOFTMAX; c.renormalize = 1; c.routed_scale = 1.0f;
  c.bias_mode = MOE_BIAS_LOGIT; c.act_dtype = MOE_BF16; c.weight_dtype = MOE_BF16;
  return c;
}
#define EXPECT(cond, code) do { if (!(cond)) { printf("failed: %s\n", #cond); return code; } } while (0)
int main(void) {
  EXPECT(moe_abi_version() == MOE_ABI_VERSION, 10);
  for (int s = 0; s <= 8; ++s) EXPECT(moe_status_str((moe_status_t)s) != NULL, 11);
  moe_layer_t h = NULL;
  /* each invalid field alone */
  struct { int field; float f; int v; moe_status_t want; } bad[] = {
    {0, 0, 0, MOE_ERR_SHAPE}, {1, 0, 17, MOE_ERR_SHAPE}, {2, 0, 513, MOE_ERR_SHAPE},
    {3, 0, 100, MOE_ERR_SHAPE}, {4, 0, 48, MOE_ERR_SHAPE}, {5, 0, -32, MOE_ERR_SHAPE},
    {6, 0, 0, MOE_ERR_SHAPE}, {7, 0, 2, MOE_ERR_DTYPE}, {8, 0, 0, MOE_ERR_DTYPE},
    {9, 0, 5, MOE_ERR_DTYPE}, {10, 0, 2, MOE_ERR_DTYPE}, {11, 0.0f, 0, MOE_ERR_SHAPE},
    {12, -1.0f, 0, MOE_ERR_SHAPE}, {13, INFINITY, 0, MOE_ERR_SHAPE}, {14, NAN, 0, MOE_ERR_SHAPE},
    {15, 0, 64, MOE_ERR_SHAPE}, {16, 0, (1 << 18) + 1, MOE_ERR_SHAPE},
  };
  for (unsigned i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    moe_layer_config_t c = base();
    switch (bad[i].field) {
      case 0: c.top_k = 0; break;
      case 1: c.top_k = bad[i].v; break;
      case 2: c.num_experts = bad[i].v; break;
      case 3: c.hidden = bad[i].v; break;
      case 4: c.inter = bad[i].v; break;
      case 5: c.shared_inter = bad[i].v; break;
      case 6: c.max_tokens = 0; break;
      case 7: c.act_dtype = bad[i].v; break;
      case 8: c.weight_dtype = 9; break;
      case 9: c.score = bad[i].v; break;
      case 10: c.bias_mode = bad[i].v; break;
      case 11: c.routed_scale = bad[i].f; break;
      case 12: c.swiglu_limit = bad[i].f; break;
      case 13: c.swiglu_limit_shared = bad[i].f; break;
      case 14: c.swiglu_limit = bad[i].f; break;
      case 15: c.weight_dtype = MOE_INT4_G32; c.inter = bad[i].v; break;
      case 16: c.max_tokens = bad[i].v; break;
    }
    moe_status_t st = moe_layer_create(&c, 0, &h);
    if (st != bad[i].want || h != NULL || moe_last_error()[0] == 0) {
      printf("case %u: status %d want %d (%s)\n", i, st, bad[i].want, moe_last_error());
      return 20;
    }
  }
  /* a valid configuration on a host without a GPU */
  moe_layer_config_t c = base();
  EXPECT(moe_layer_create(&c, 0, &h) == MOE_ERR_DEVICE && h == NULL, 30);
  EXPECT(strlen(moe_last_error()) > 0, 31);
  /* NULL handles and pointers everywhere */
  EXPECT(moe_layer_create(NULL, 0, &h) == MOE_ERR_NULL, 40);
  EXPECT(moe_layer_create(&c, 0, NULL) == MOE_ERR_NULL, 41);
  moe_layer_destroy(NULL);
  EXPECT(moe_layer_packed_bytes(NULL) == 0, 42);
  EXPECT(moe_layer_workspace_bytes(NULL, 8) == 0, 43);
  EXPECT(moe_layer_pack_weights(NULL, NULL, NULL, NULL) == MOE_ERR_NULL, 44);
  moe_route_t r;
  EXPECT(moe_layer_forward(NULL, 4, NULL, NULL, NULL, NULL, NULL, NULL, 0, &r, NULL) == MOE_ERR_NULL, 45);
  EXPECT(moe_layer_forward_noalloc(NULL, 4, NULL, NULL, NULL, NULL, NULL, &r, NULL) == MOE_ERR_NULL, 46);
  EXPECT(moe_layer_forward_timed(NULL, 4, NULL, NULL, NULL, NULL, NULL, NULL, 0, &r, NULL, NULL) == MOE_ERR_NULL, 47);
  EXPECT(moe_debug_checks() == 0, 48);
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm clang")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    objdir = os.path.join(PKG, "lib", "obj")
    kernels = [os.path.join(objdir, n + ".o") for n in
               ("moe_router", "moe_dispatch", "moe_gemm_stream", "moe_gemm_tiled", "moe_combine",
                "moe_pack")]
    if not all(os.path.exists(o) for o in kernels):
        pytest.skip("release objects not built")
    san_host = []
    for s in SAN:   # host code only: each sanitizer flag applies to the host pass
        san_host += ["-Xarch_host", f"-fsanitize={s}"]
    san_host += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
    abi_o = str(tmp_path / "moe_abi_san.o")
    cc = subprocess.run([HIPCC, "-x", "hip", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-O1",
                         "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature",
                         "-Xclang", "-packed-fp32-ops", *san_host, "-c",
                         os.path.join(PKG, "csrc", "moe_abi.cpp"), "-o", abi_o],
                        capture_output=True, text=True, timeout=600)
    assert cc.returncode == 0, cc.stderr[-3000:]
    lib = str(tmp_path / "libmoe_san.so")
    ln = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *kernels, abi_o,
                         "-o", lib], capture_output=True, text=True, timeout=600)
    assert ln.returncode == 0, ln.stderr[-3000:]
    src = tmp_path / "driver.c"
    src.write_text(DRIVER)
    exe = str(tmp_path / "driver")
    drv = subprocess.run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined",
                          "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
                          f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
                          str(src), "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", "-lm"],
                         capture_output=True, text=True, timeout=300)
    assert drv.returncode == 0, drv.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert run.stdout.strip().endswith("ok")
