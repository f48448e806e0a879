"""Build the HIP library ``libattn.so`` for gfx950 with hipcc.

Every source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into ``exact_attention_25_amd/libattn.so``.  The
library exports the C ABI declared in ``include/attn.h``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep fp32 arithmetic in plain (non-packed) VALU forms.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wno-unused-command-line-argument",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


# The 16-bit backward kernels keep their MFMA results in VGPRs and their
# long-lived operand fragments in AGPRs (pin_agpr in attn_bwd_kernel.h);
# without this the compiler gives every MFMA an AGPR result once a kernel
# needs AGPRs, and the vector code then copies S and dP out element by
# element (measured: causal GQA backward -4 %, soft-capped ViT -18 %).
FILE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
for _v in ("bf16_d64", "bf16_d128", "fp16_d64", "fp16_d128"):
    FILE_FLAGS[f"attn_bwd_var_{_v}.hip"] = FILE_FLAGS["attn_bwd.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ([hipcc()] + HIP_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + list(extra)
           + ["-c", src, "-o", obj])
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
