"""Build libtsoftmax.so in-tree for gfx950 with hipcc.

    python -m temperature_softmax_vocabulary_amd.build [--verbose]

Compiles every source under csrc/ to an object in _build/ and links the shared
library next to this file. Always rebuilds (the sources are small).

It also links libtsoftmax_noguard.so from the same sources with TS_NO_INF_GUARD:
the arithmetic without the -inf guard, loaded only by the tests that show what
the guard changes (nothing on finite rows; NaN rows without it).
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtsoftmax.so")
LIB_NOGUARD = os.path.join(HERE, "libtsoftmax_noguard.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
SOURCES = ["softmax_kernels.hip", "draw_kernels.hip", "measure_kernels.hip", "tsoftmax_api.cpp"]

# -ffast-math and friends are never used: -inf and NaN semantics are the point.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # every floating-point operation exactly as written (no a*b+c fusion): the
    # -inf guard must be a pure select, bit for bit on finite rows
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtsoftmax)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _link(cc, objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)


def _compile_cmd(cc, subdir, defines, src):
    out = os.path.join(BUILD, subdir)
    os.makedirs(out, exist_ok=True)
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    return obj, [cc, *COMMON, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    flavours = [("release", [], LIB), ("noguard", ["-DTS_NO_INF_GUARD"], LIB_NOGUARD)]
    jobs = {name: [_compile_cmd(cc, name, defs, src) for src in SOURCES] for name, defs, _ in flavours}
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for js in jobs.values() for _, cmd in js]:
            f.result()
    for name, _, lib in flavours:
        _link(cc, [obj for obj, _ in jobs[name]], lib, verbose)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose)
    print(f"built {path}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
