"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into
``libfa_mi355x.so`` next to this file (in-tree, so it travels with the repo).

Usage:  python -m io_aware_exact_fa1_amd.build   (or call ``build()``).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "fa_fwd.hip")
SRC_BWD = os.path.join(HERE, "csrc", "fa_bwd.hip")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_fwd_f32.hip", "fa_split.hip", "fa_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_cmd(out, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU ops stay off: plain fp32 ops only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *extra, *SOURCES, "-o", out,
    ]


def build(verbose=False):
    tmp = LIB_PATH + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
