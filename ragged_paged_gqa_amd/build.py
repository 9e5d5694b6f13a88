"""Build the HIP library (gfx950) in-tree: ragged_paged_gqa_amd/_build/librpa.so."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# the kernels and the C entry points that launch them; the host logic that
# touches no device (also built without HIP by the sanitizer test)
SRC = os.path.join(HERE, "csrc", "rpa_api.hip")
HOST_SRC = os.path.join(HERE, "csrc", "rpa_host.cpp")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "librpa.so")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
    ]


def build(verbose: bool = False, out: str | None = None, defines: tuple[str, ...] = ()) -> str:
    """Compile librpa.so (or `out`); `defines` are NAME=VALUE tuning overrides."""
    lib = out or LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [hipcc(), *compile_flags(), *(f"-D{d}" for d in defines), "-o", tmp, SRC, HOST_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    print(build(verbose=True, out=a.out, defines=tuple(a.defines)))
