"""Build libattn.so (the HIP/gfx950 kernels and the C ABI) in-tree with hipcc,
and libattn_probe.so (the dense MFMA loop the benchmark reports beside the
published peaks; not part of the attention path or its ABI).

Any compiler warning fails the build (the host pass's notice that it does not
know the packed-fp32 target feature aside).

Usage: python -m bit_quantized_exact_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libattn.so")
PROBE_OUT = os.path.join(HERE, "libattn_probe.so")
PROBE_SRC = os.path.join(HERE, "probe", "mfma_probe.hip")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    # never emit packed fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]
# Per-file flags: the quantisation kernels must not fuse products (bit-exact contract).
SOURCES = {
    "attn_quant.hip": ["-ffp-contract=off"],
    "attn_fwd.hip": [],
    "attn_decode.hip": [],
    "attn_api.hip": [],
}


def _compile(src: str, extra: list[str]) -> str:
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *extra, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        # e.g. -Winline-asm: an asm block listing a register the compiler reserves
        raise RuntimeError(f"hipcc warned for {src} (warnings fail the build):\n{msgs}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = list(SOURCES.items()) + [(PROBE_SRC, ["-I", os.path.dirname(PROBE_SRC)])]
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), jobs))
    _link(objs[:-1], OUT)
    _link(objs[-1:], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
