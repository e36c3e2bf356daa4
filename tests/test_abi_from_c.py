"""The C ABI from C: a C11 program that includes include/moe_layer.h, links the
library directly (no Python, no torch) and calls entry points that answer
without a GPU (version, status names, argument validation)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_mixture_experts_layer_amd", "lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SRC = r"""
#include "moe_layer.h"
#include <stdio.h>
#include <string.h>
int main(void) {
  if (moe_abi_version() != MOE_ABI_VERSION) return 10;
  if (strcmp(moe_status_str(MOE_ERR_WORKSPACE), "MOE_ERR_WORKSPACE") != 0) return 11;
  moe_layer_config_t c;
  memset(&c, 0, sizeof c);
  c.hidden = 256; c.num_experts = 16; c.top_k = 2; c.inter = 64; c.shared_inter = 64;
  c.max_tokens = 64; c.score = MOE_SCORE_SOFTMAX; c.renormalize = 1; c.routed_scale = 1.0f;
  c.bias_mode = MOE_BIAS_LOGIT; c.act_dtype = MOE_BF16; c.weight_dtype = MOE_BF16;
  c.top_k = 17;                                  /* invalid: more than 16 */
  moe_layer_t h = NULL;
  moe_status_t st = moe_layer_create(&c, 0, &h);
  if (st != MOE_ERR_SHAPE || h != NULL || strstr(moe_last_error(), "top_k") == NULL) return 12;
  if (moe_layer_create(NULL, 0, &h) != MOE_ERR_NULL) return 13;
  moe_layer_destroy(NULL);                       /* ignored */
  if (moe_layer_packed_bytes(NULL) != 0 || moe_layer_workspace_bytes(NULL, 8) != 0) return 14;
  printf("ok %d\n", moe_abi_version());
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_and_library_from_c(tmp_path):
    lib = os.path.join(LIBDIR, "libmoe_mi355x.so")
    assert os.path.exists(lib), "library not built"
    src = tmp_path / "abi.c"
    src.write_text(SRC)
    exe = tmp_path / "abi"
    cc = subprocess.run(
        ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
         "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
         f"-I{os.path.join(ROCM, 'include')}", str(src), "-o", str(exe), f"-L{LIBDIR}",
         "-lmoe_mi355x", f"-Wl,-rpath,{LIBDIR}"],
        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.strip() == "ok 3"
