"""Build libtsa.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m token_sparse_attention_rel_amd.build [--jobs N] [--debug]

Every source under csrc/ is compiled to an object under _build/ and linked
into token_sparse_attention_rel_amd/libtsa.so.  hipcc cross-compiles, so this
runs on a machine without a GPU.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtsa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtsa)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def flags(debug: bool = False) -> list[str]:
    f = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-fPIC",
        "-O3",
        "-Wall",
        "-Wno-unused-function",
        # keep packed-fp32 instructions out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(ROOT, 'include')}",
        f"-I{CSRC}",
    ]
    if debug:
        f += ["-g", "-DTSA_DEBUG=1"]
    return f


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *flags(debug), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--debug", action="store_true")
    args = ap.parse_args(argv)
    build(args.jobs, args.debug, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
