"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into
``libfa_mi355x.so`` next to this file (in-tree, so it travels with the repo).

Each source is compiled to its own object in parallel, then the objects are
linked into the shared library.

Usage:  python -m io_aware_exact_fa1_amd.build   (or call ``build()``).
        python -m io_aware_exact_fa1_amd.build --out PATH -D FA_D64_BC=64 -D FA_D64_NW=4
            builds a tile-shape variant elsewhere (B_c keys per K/V tile and
            NW waves of 32 query rows, per head dimension); the binding loads
            it when FA_MI355X_LIB names it.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("fa_fwd.hip", "fa_fwd_f32.hip", "fa_split.hip", "fa_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops stay off: plain fp32 ops only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *extra,
    ]


def compile_cmd(out, extra=()):
    """One hipcc command that compiles every source and links the library."""
    return [hipcc(), *compile_flags(extra), "-shared", *SOURCES, "-o", out]


def _filter(stderr):
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    return [ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln]


def build(verbose=False, extra=(), out=None, sources=None):
    """Compile ``sources`` (default: every source) with ``extra`` flags and
    link them into ``out`` (default: the library next to this file)."""
    out = out or LIB_PATH
    sources = sources or SOURCES
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in sources]
        cmds = [[hipcc(), *compile_flags(extra), "-c", s, "-o", o] for s, o in zip(sources, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
        errs = []
        for c, r in zip(cmds, results):
            e = _filter(r.stderr)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {c[-3]}:\n" + "\n".join(e))
            errs += e
        tmp = out + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_filter(r.stderr)))
        if verbose and errs:
            print("\n".join(errs), file=sys.stderr)
        os.replace(tmp, out)
        return out
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description="build the HIP library for gfx950")
    ap.add_argument("--out", default=None, help="library path (default: next to this file)")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="preprocessor definition, e.g. FA_D64_BC=64 (tile-shape variants)")
    a = ap.parse_args(argv)
    out = a.out
    if out:
        os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    print(build(verbose=True, extra=[f"-D{x}" for x in a.defines], out=out))


if __name__ == "__main__":
    main()
