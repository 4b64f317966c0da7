"""Build libtsa.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m token_sparse_attention_rel_amd.build [--jobs N] [--debug | --sanitize]

Every source under csrc/ is compiled to an object under _build/ and linked
into token_sparse_attention_rel_amd/libtsa.so.  hipcc cross-compiles, so this
runs on a machine without a GPU.

  --debug     token_sparse_attention_rel_amd/libtsa_debug.so, built with TSA_DEBUG:
              every index list is checked (in range, strictly increasing) before a
              kernel reads it, and a violation returns TSA_ERR_SHAPE.
  --sanitize  _build/san/libtsa_san.so, the host code built with AddressSanitizer and
              UndefinedBehaviorSanitizer (the device code as usual), for running the
              host-side argument validation under the sanitizers: load it with
              TSA_LIB=<path> and the clang ASan runtime preloaded.
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
LIB_DEBUG = os.path.join(PKG, "libtsa_debug.so")
LIB_SAN = os.path.join(BUILD, "san", "libtsa_san.so")
ARCH = "gfx950"

VARIANTS = {
    # name: (object directory, library, extra compile flags, extra link flags)
    "release": (BUILD, LIB, [], []),
    "debug": (os.path.join(BUILD, "debug"), LIB_DEBUG, ["-DTSA_DEBUG=1"], []),
    "sanitize": (os.path.join(BUILD, "san"), LIB_SAN,
                 ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"],
                 ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]),
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtsa)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def flags(extra=()) -> list[str]:
    return [
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
        *extra,
    ]


def _compile(src: str, objdir: str, extra) -> str:
    obj = os.path.join(objdir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *flags(extra), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, debug: bool = False, verbose: bool = False, variant: str | None = None) -> str:
    """Compile and link one variant ('release', 'debug' or 'sanitize'); returns the library path."""
    variant = variant or ("debug" if debug else "release")
    objdir, lib, cflags, lflags = VARIANTS[variant]
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, cflags), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *lflags, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources ({variant})")
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    g = ap.add_mutually_exclusive_group()
    g.add_argument("--debug", action="store_true")
    g.add_argument("--sanitize", action="store_true")
    args = ap.parse_args(argv)
    variant = "debug" if args.debug else ("sanitize" if args.sanitize else "release")
    build(args.jobs, verbose=True, variant=variant)
    return 0


if __name__ == "__main__":
    sys.exit(main())
