"""Build libmaskmods.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m mask_mods_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles. Objects go to ``mask_mods_amd/_build/``; the library is
written atomically to ``mask_mods_amd/libmaskmods.so``.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmaskmods.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

SOURCES = [
    "api.cpp",
    "fwd_bf16_d128.hip",
    "fwd_bf16_d64.hip",
    "fwd_f16_d128.hip",
    "fwd_f16_d64.hip",
    "fwd_fp8_d128.hip",
    "fwd_fp8_d64.hip",
    "fwd_f32.hip",
    "decode.hip",
    "block_mask.hip",
    "bwd.hip",
    "bwd_bf16_d128.hip",
    "bwd_bf16_d64.hip",
    "bwd_f16_d128.hip",
    "bwd_f16_d64.hip",
]


def source_hash() -> str:
    """Hash of every kernel, ABI and header source the library is built from (16 hex
    digits). The build stamps it into the library; the binding compares the two at load,
    so a library left over from other sources is refused instead of run."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if os.path.splitext(name)[1] in (".hip", ".h", ".cpp"):
                h.update(name.encode() + b"\0")
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
                h.update(b"\0")
    return h.hexdigest()[:16]


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    log = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if log:
        sys.stderr.write(f"[{src}]\n" + "\n".join(log) + "\n")
    return obj


def build(jobs: int | None = None, resource_usage: bool = False, out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link ``out`` (``resource_usage``: print each kernel's
    register, LDS and spill figures)."""
    os.makedirs(build_dir, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    extra += [f"-DMM_SOURCE_HASH=\"{source_hash()}\""]
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(resource_usage="--usage" in sys.argv))
