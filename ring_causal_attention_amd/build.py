"""Builds liblwm_attn.so (HIP for gfx950) in-tree with hipcc.

Run ``python -m ring_causal_attention_amd.build`` (or ``__graft_entry__.build()``).  Each source is
compiled to an object in ``_build/`` and linked into ``ring_causal_attention_amd/liblwm_attn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblwm_attn.so")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "profile.cpp", "rope.hip", "attn_fwd.hip", "attn_bwd.hip", "ffn.hip", "probe.hip"]

# Packed-FP32 VALU forms are disabled for device code; the host pass ignores the feature.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return h


# Per-source code-generation options.  The backward's dK/dV kernel keeps 128 fp32 accumulators
# live across its loop; with MFMA results in VGPRs the register allocator spills rarely used values
# to AGPRs instead of copying the accumulators between the two files every iteration.
SOURCE_FLAGS = {"attn_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra=(), bdir: str = BUILD) -> str:
    os.makedirs(bdir, exist_ok=True)
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Host-side AddressSanitizer for the checking build (device code is built as usual).
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = True, save_temps: bool = False, host_asan: bool = False) -> str:
    """Compile and link the library.  With host_asan the host code (argument checks, timing) is
    instrumented by AddressSanitizer and the library goes to _build/asan/liblwm_attn.so instead
    of the package; load it with LWM_ATTN_LIB and the sanitizer runtime preloaded."""
    extra = ["-save-temps=obj"] if save_temps else []
    bdir, out = BUILD, LIB
    if host_asan:
        extra = extra + HOST_ASAN
        bdir = os.path.join(BUILD, "asan")
        out = os.path.join(bdir, "liblwm_attn.so")
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, bdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *(HOST_ASAN if host_asan else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(save_temps="--save-temps" in sys.argv, host_asan="--host-asan" in sys.argv)


# Kernel sources per family of kernels: a counter record taken on one family stays valid while
# only another family's sources change.
KERNEL_FAMILIES = {"attention": ["rope.hip", "attn_fwd.hip", "attn_bwd.hip"], "ffn": ["ffn.hip"]}


def sources_digest(family: str | None = None) -> str:
    """sha256 over the device headers and the kernel sources of `family` (all kernels when None):
    identifies the code a measurement was taken on."""
    import hashlib
    hsh = hashlib.sha256()
    hip = sorted(n for n in os.listdir(CSRC) if n.endswith(".hip"))
    if family is not None:
        hip = [n for n in hip if n in KERNEL_FAMILIES[family]]
    names = sorted(n for n in os.listdir(CSRC) if n.endswith(".hpp")) + hip
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            hsh.update(n.encode() + b"\0" + f.read())
    return hsh.hexdigest()
