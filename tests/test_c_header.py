"""include/lwm_attn.h is a C header: a C99 program that includes it compiles with warnings as
errors, links against the built library and runs its host-side paths (no GPU needed: the calls
below fail validation, or only size a workspace, before anything is launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ring_causal_attention_amd")
LIB = os.path.join(PKG, "liblwm_attn.so")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "lwm_attn.h"

int main(void) {
  if (lwm_abi_version() != LWM_ABI_VERSION) { printf("version %d\n", lwm_abi_version()); return 1; }
  /* a NULL tensor descriptor is rejected on the host with a message */
  lwm_tensor4 q;
  memset(&q, 0, sizeof q);
  q.dtype = LWM_BF16; q.B = 1; q.L = 4; q.H = 1; q.D = 128; q.sB = 512; q.sL = 128; q.sH = 128;
  int st = lwm_blockattn_fwd(&q, NULL, NULL, NULL, NULL, 0, 0, 1, 0.0f, NULL, NULL, NULL);
  if (st != LWM_ERR_INVALID_ARG || strlen(lwm_last_error()) == 0) { printf("fwd status %d\n", st); return 2; }
  /* an unsupported head dimension is refused as such */
  q.D = 64; q.sB = 256; q.sL = 64; q.sH = 64;
  lwm_tensor4 o = q;
  float* lse = NULL;
  st = lwm_blockattn_fwd(&q, &q, &q, NULL, NULL, 0, 0, 1, 0.0f, &o, lse, NULL);
  if (st >= 0) { printf("D=64 accepted\n"); return 3; }
  size_t ws = lwm_blockattn_bwd_workspace_size(2, 3, 100, 100, 128);
  if (ws < (size_t)2 * 2 * 3 * 100 * sizeof(float)) { printf("workspace %zu\n", ws); return 4; }
  printf("ok %s\n", lwm_last_error());
  return 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(LIB):
        pytest.skip("library not built (run __graft_entry__.build())")
    src = tmp_path / "use_header.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_header"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", PKG, "-llwm_attn", f"-Wl,-rpath,{PKG}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok")
