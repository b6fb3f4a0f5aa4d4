"""The oracle's native twin: ``tiled_ref.c`` (plain C, fp64) through ctypes.

TEST INFRASTRUCTURE ONLY (see ``oracle/ref.py``).  Only the test suite and
the CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
library: the C file is compiled with the host compiler (gcc) into its own
shared object next to it, never linked with the library.

  * ``build_native()``   - compile ``tiled_ref.c`` (always, e.g. from the
                           build step); returns the library path.
  * ``tiled_ref_c(q, k, v, scale, causal, Br, Bc)`` - the recurrence on
                           [..., N, d] arrays, the same contract as
                           ``oracle.tiled_ref`` (O, LSE in float64).
  * ``tiled_rows_c(q, k, v, scale, causal, Br, Bc, row0, row1)`` - query
                           rows row0 .. row1-1 of one head ([N, d] arrays).
"""

import ctypes
import os
import shutil
import subprocess
import tempfile
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "tiled_ref.c")
LIB = os.path.join(HERE, "libfa_oracle_c.so")

_lock = threading.Lock()
_lib = None


def compile_c(source, out):
    """gcc -O2 (IEEE arithmetic: no fast-math) into a shared object."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc) to build the C oracle")
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([cc, "-O2", "-std=c99", "-fPIC", "-shared", source, "-o", tmp, "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C oracle failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


def build_native():
    return compile_c(SOURCE, LIB)


def load(path=None):
    """The compiled C oracle (built first when missing or older than its source)."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SOURCE):
                build_native()
            _lib = _bind(ctypes.CDLL(LIB))
        return _lib


def _bind(lib):
    f = lib.fa_oracle_tiled_rows
    dp = ctypes.POINTER(ctypes.c_double)
    f.argtypes = [dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_long, ctypes.c_double, ctypes.c_int,
                  ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long]
    f.restype = ctypes.c_int
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def tiled_rows_c(q, k, v, scale, causal, Br, Bc, row0, row1, lib=None, out=None):
    """Rows row0 .. row1-1 of one head; returns (O rows, LSE rows).  ``out``
    may pass preallocated full-size (o, lse) arrays to write into."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    n, d = q.shape
    if k.shape != (n, d) or v.shape != (n, d):
        raise ValueError("q, k, v must all be [N, d]")
    o, lse = out if out is not None else (np.zeros((n, d)), np.zeros(n))
    st = lib.fa_oracle_tiled_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), n, d, float(scale),
                                  int(bool(causal)), int(Br), int(Bc), int(row0), int(row1))
    if st == -1:
        raise ValueError("a query row has no visible key")
    if st != 0:
        raise ValueError("bad arguments to the C oracle (status %d)" % st)
    return o[row0:row1], lse[row0:row1]


def tiled_ref_c(q, k, v, scale, causal, Br, Bc, lib=None):
    """The recurrence over every head of [..., N, d] inputs."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf, kf, vf = (np.ascontiguousarray(x.reshape(-1, n, d)) for x in (q, k, v))
    o = np.zeros_like(qf)
    lse = np.zeros(qf.shape[:2])
    for g in range(qf.shape[0]):
        tiled_rows_c(qf[g], kf[g], vf[g], scale, causal, Br, Bc, 0, n, lib=lib, out=(o[g], lse[g]))
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)


def mutant_library(replacements):
    """A copy of the C oracle with textual replacements, compiled into a
    temporary directory (planted mistakes for the mutant tests); returns the
    loaded library.  Each replacement must match the source exactly once."""
    with open(SOURCE) as f:
        src = f.read()
    for old, new in replacements:
        if src.count(old) != 1:
            raise ValueError("replacement target must occur once: %r" % old)
        src = src.replace(old, new)
    tmpdir = tempfile.mkdtemp(prefix="fa_oracle_mutant_")
    path = os.path.join(tmpdir, "mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib_path = compile_c(path, os.path.join(tmpdir, "libmutant.so"))
    return _bind(ctypes.CDLL(lib_path))
