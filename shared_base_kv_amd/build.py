"""Build the HIP library liblra.so in-tree for gfx950 (hipcc cross-compiles
without a GPU). Usage: python -m shared_base_kv_amd.build"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblra.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_*_f32 anywhere (they are not used by this library).
# kernarg preload: a kernel's leading scalar and pointer arguments, up to 14
# dwords, arrive in SGPRs at wave start (the decode kernel's work-item fields);
# a kernel whose first argument is a struct preloads nothing.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["lra_api.cpp", "decode_bf16.hip", "decode_bf16_kv.hip", "decode_f32.hip", "lr_build.hip", "prefill_bf16.hip"]


DEBUG_OUT = os.path.join(HERE, "liblra_debug.so")
# the debug library: the same kernels, with the API layer built to check the
# device-side inputs before each attention launch
DEBUG_SOURCE = ("lra_api.cpp", "lra_api_debug", ["-DLRA_DEBUG_CHECKS"])


def _compile(spec) -> str:
    src, stem, extra = (spec, os.path.splitext(spec)[0], []) if isinstance(spec, str) else spec
    obj = os.path.join(BUILD_DIR, stem + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, [*SOURCES, DEBUG_SOURCE]))
    debug_obj = objs.pop()
    for out, api_obj in ((OUT, objs[0]), (DEBUG_OUT, debug_obj)):
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_obj, *objs[1:], "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, out)
        if verbose:
            print(f"built {out}")
    return OUT


if __name__ == "__main__":
    build()
