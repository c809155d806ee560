"""Build libattn.so (the product) and libattn_probes.so (test-only probes) for gfx950.

Both libraries are built in-tree next to this file with hipcc.  Every HIP
source is compiled with packed-fp32 VALU instructions switched off.

Run:  python -m exact_attention_forward_tiled_amd.build
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", CSRC, "-I", os.path.join(ROOT, "include")]

LIBS = {
    "libattn.so": ["attn_api.cpp", "attn_fwd_bf16.hip", "attn_mxfp4.hip", "attn_mxfp8.hip",
                   "attn_bwd_bf16.hip"],
    "libattn_probes.so": ["probes.hip"],
}


def _compile(src):
    os.makedirs(OBJ, exist_ok=True)
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = (["-x", "hip"] if src.endswith(".hip")
            else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")])
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def build(verbose=False):
    """Compile every source and link both shared libraries; returns their paths."""
    sources = sorted({s for srcs in LIBS.values() for s in srcs})
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = dict(zip(sources, ex.map(_compile, sources)))
    outs = []
    for lib, srcs in LIBS.items():
        target = os.path.join(HERE, lib)
        tmp = target + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [objs[s] for s in srcs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, target)
        outs.append(target)
        if verbose:
            print("built", target)
    return outs


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
