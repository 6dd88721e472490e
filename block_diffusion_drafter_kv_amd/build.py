"""Build the HIP library libdflash_amd.so in-tree for gfx950 (hipcc, no JIT)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdflash_amd.so")
SOURCES = ["api.hip", "kernels.hip", "attention.hip", "gemm_bf16.hip", "gemm_f16.hip", "gemm_f32.hip",
           "noalloc.hip"]
ARCH = os.environ.get("DFLASH_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = True, jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        rc, out = _run([_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return src, obj, rc, out

    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    failed = [(s, o) for s, _, rc, o in results if rc != 0]
    for s, _, rc, o in results:
        if verbose and o.strip():
            print(f"[{s}]\n{o}", file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed) + "\n" +
                           "\n".join(o for _, o in failed))
    tmp = LIB + ".tmp"
    rc, out = _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
                    *[o for _, o, _, _ in results]])
    if rc != 0:
        raise RuntimeError("link failed:\n" + out)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
