"""ctypes binding of the C ABI in ``include/fa.h`` (argument marshalling only).

The functions ``fa_fwd``, ``fa_fwd_f32``, ``fa_fwd_ex``, ``fa_fwd_split``,
``fa_fwd_split_noalloc``, ``fa_bwd``, ``fa_strerror``, ``fa_check_args``, ``fa_check_args_ex``,
``fa_check_args_split``, ``fa_split_chunks`` and ``fa_bwd_check_args`` have
the names and argument order of the C entry points; tensors are passed
as their device pointers and streams as HIP stream handles.  Every step of
the computation runs in the HIP library: there is no fallback path, and a
missing or unloadable library raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEAD_DIM = 3
FA_ERR_SCALE = 4
FA_ERR_ALIAS = 5
FA_ERR_LAUNCH = 6
FA_ERR_ALIGN = 7
FA_ERR_VARIANT = 8
FA_ERR_SCRATCH = 9
FA_SPLIT_NOALLOC_BYTES = 32 << 20
FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1

EXPORTED = ("fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_fwd_split", "fa_fwd_split_noalloc", "fa_bwd", "fa_strerror",
            "fa_supported",
            "fa_check_args", "fa_check_args_ex", "fa_check_args_split", "fa_split_chunks", "fa_bwd_check_args")

_lib = None


class FaError(RuntimeError):
    """A nonzero status returned by the HIP library."""

    def __init__(self, status, where):
        self.status = int(status)
        super().__init__(f"{where}: status {status}: {fa_strerror(status)}")


def load_library(path=None):
    """Load the HIP library (once).  torch is imported first so that the
    library binds to the HIP runtime torch already loaded.  The library is
    the one built next to this file, or the build that the environment
    variable FA_MI355X_LIB names (e.g. a tile-shape variant)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (must precede the CDLL: one HIP runtime per process)
    p = path or os.environ.get("FA_MI355X_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"HIP library {p} is not built: run `python -m io_aware_exact_fa1_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(p)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.argtypes = sig
    lib.fa_fwd.restype = i
    lib.fa_fwd_f32.argtypes = sig
    lib.fa_fwd_f32.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_supported.argtypes = [i, i]
    lib.fa_supported.restype = i
    lib.fa_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i]
    lib.fa_check_args.restype = i
    lib.fa_fwd_ex.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_ex.restype = i
    lib.fa_check_args_ex.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, i]
    lib.fa_check_args_ex.restype = i
    lib.fa_fwd_split.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, i, i, vp, vp, vp]
    lib.fa_fwd_split.restype = i
    lib.fa_fwd_split_noalloc.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, i, i, vp]
    lib.fa_fwd_split_noalloc.restype = i
    lib.fa_check_args_split.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, i, i, vp, vp]
    lib.fa_check_args_split.restype = i
    lib.fa_split_chunks.argtypes = [i, i]
    lib.fa_split_chunks.restype = i
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_check_args.argtypes = [vp] * 10 + [i, i, i, i, f, i]
    lib.fa_bwd_check_args.restype = i
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    """C ``fa_fwd``: bf16 q, k, v, o and fp32 lse; returns the status code."""
    return load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N),
                                 int(d), float(scale), int(causal), _stream(stream))


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    """C ``fa_fwd_f32``: fp32 q, k, v, o and lse; returns the status code."""
    return load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                     int(N), int(d), float(scale), int(causal), _stream(stream))


def fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, stream=None):
    """C ``fa_fwd_ex``: bf16 q, o [B, Hq, T, d], k, v [B, Hkv, S, d], fp32 lse."""
    return load_library().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq), int(Hkv),
                                    int(T), int(S), int(d), float(scale), int(causal), int(offset), int(window),
                                    _stream(stream))


def fa_fwd_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, ws_o, ws_lse,
                 stream=None):
    """C ``fa_fwd_split``: as ``fa_fwd_ex`` plus nsplit and the fp32
    workspaces ws_o [G, B, Hq, T, d] and ws_lse [G, B, Hq, T]."""
    return load_library().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq), int(Hkv),
                                       int(T), int(S), int(d), float(scale), int(causal), int(offset), int(window),
                                       int(nsplit), _ptr(ws_o), _ptr(ws_lse), _stream(stream))


def fa_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, stream=None):
    """C ``fa_fwd_split_noalloc``: ``fa_fwd_split`` with its partials in the
    library's static device scratch (no workspaces, nothing allocated)."""
    return load_library().fa_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
                                               int(Hkv), int(T), int(S), int(d), float(scale), int(causal),
                                               int(offset), int(window), int(nsplit), _stream(stream))


def fa_check_args_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, ws_o,
                        ws_lse):
    return load_library().fa_check_args_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
                                              int(Hkv), int(T), int(S), int(d), float(scale), int(causal),
                                              int(offset), int(window), int(nsplit), _ptr(ws_o), _ptr(ws_lse))


def fa_split_chunks(S, nsplit):
    """Number of key chunks G that ``fa_fwd_split`` uses."""
    return load_library().fa_split_chunks(int(S), int(nsplit))


def fa_check_args_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window):
    return load_library().fa_check_args_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
                                           int(Hkv), int(T), int(S), int(d), float(scale), int(causal),
                                           int(offset), int(window))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream=None):
    """C ``fa_bwd``: bf16 q, k, v, o, dout, dq, dk, dv; fp32 lse and delta."""
    return load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(delta), int(B), int(H), int(N), int(d),
                                 float(scale), int(causal), _stream(stream))


def fa_bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal):
    return load_library().fa_bwd_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), int(B), int(H),
                                            int(N), int(d), float(scale), int(causal))


def fa_strerror(status):
    return load_library().fa_strerror(int(status)).decode()


def fa_supported(d, dtype):
    """1 if the library takes head dimension d with FA_DTYPE_BF16 / FA_DTYPE_F32 inputs, else 0."""
    return int(load_library().fa_supported(int(d), int(dtype)))


def fa_check_args(q, k, v, o, lse, B, H, N, d, scale, causal, elem_bytes):
    return load_library().fa_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                        int(N), int(d), float(scale), int(causal), int(elem_bytes))


def _one_device(*ts):
    dev = ts[0].device
    if any(t.device != dev for t in ts):
        raise ValueError("all tensors must be on one GPU")


def _check_out(t, shape, dtype, device, name):
    """A caller-supplied output buffer must be exactly what the C entry point
    writes: it trusts the buffer sizes it is given."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")


def forward(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """Allocate O / LSE with torch (if not given), call the C entry point for
    the dtype of q, raise FaError on a nonzero status; returns (O, LSE).

    q, k, v: CUDA tensors [B, H, N, d] of one dtype (bfloat16 or float32).
    """
    import math
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 4:
        raise ValueError("q, k and v must share one [B, H, N, d] shape")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k and v must share one dtype")
    _one_device(q, k, v)
    B, H, N, d = q.shape
    q, k, v = (x.contiguous() for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q.shape, q.dtype, q.device, "out")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    with torch.cuda.device(q.device):
        if q.dtype == torch.bfloat16:
            st = fa_fwd(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
            where = "fa_fwd"
        elif q.dtype == torch.float32:
            st = fa_fwd_f32(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
            where = "fa_fwd_f32"
        else:
            raise ValueError(f"unsupported dtype {q.dtype}")
    if st != FA_OK:
        raise FaError(st, where)
    return out, lse


def backward(q, k, v, o, lse, dout, causal=False, scale=None, stream=None):
    """Allocate dQ, dK, dV and the D workspace with torch, call ``fa_bwd``,
    raise FaError on a nonzero status; returns (dQ, dK, dV, D).

    q, k, v, o, dout: bfloat16 CUDA tensors [B, H, N, d]; lse: float32
    [B, H, N] from the forward with the same causal and scale.
    """
    import math
    import torch
    ts = (q, k, v, o, dout)
    if not all(x.is_cuda for x in ts + (lse,)):
        raise ValueError("all tensors must be GPU tensors")
    if any(x.shape != q.shape for x in ts) or q.dim() != 4:
        raise ValueError("q, k, v, o and dout must share one [B, H, N, d] shape")
    _one_device(*ts, lse)
    if any(x.dtype != torch.bfloat16 for x in ts) or lse.dtype != torch.float32:
        raise ValueError("q, k, v, o, dout must be bfloat16 and lse float32")
    B, H, N, d = q.shape
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    q, k, v, o, dout, lse = (x.contiguous() for x in (q, k, v, o, dout, lse))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv, delta


def forward_ex(q, k, v, causal=False, scale=None, offset=None, window=0, stream=None):
    """Variants of ``forward`` through ``fa_fwd_ex``: q [B, Hq, T, d] and
    k, v [B, Hkv, S, d] bfloat16 CUDA tensors (Hq a multiple of Hkv); query
    row i sits at position offset + i (default S - T) for the causal mask;
    window > 0 limits each row to the window keys ending at its position.
    Returns (O [B, Hq, T, d], LSE [B, Hq, T])."""
    import math
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, T, d] and k, v one [B, Hkv, S, d] shape")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("q, k and v must share B and d")
    if any(x.dtype != torch.bfloat16 for x in (q, k, v)):
        raise ValueError("fa_fwd_ex takes bfloat16 tensors")
    _one_device(q, k, v)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    q, k, v = (x.contiguous() for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if offset is None:
        offset = S - T
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_ex(q, k, v, out, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_ex")
    return out, lse


def forward_split(q, k, v, causal=False, scale=None, offset=None, window=0, nsplit=8, workspace=None,
                  stream=None):
    """``forward_ex`` through ``fa_fwd_split``: the keys are cut into
    G = fa_split_chunks(S, nsplit) chunks whose partial results are merged.
    ``workspace`` may be a (ws_o [G, B, Hq, T, d], ws_lse [G, B, Hq, T])
    pair of float32 CUDA tensors to use (and read back afterwards); else
    they are allocated here.  Returns (O, LSE)."""
    import math
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, T, d] and k, v one [B, Hkv, S, d] shape")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("q, k and v must share B and d")
    if any(x.dtype != torch.bfloat16 for x in (q, k, v)):
        raise ValueError("fa_fwd_split takes bfloat16 tensors")
    _one_device(q, k, v)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    q, k, v = (x.contiguous() for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if offset is None:
        offset = S - T
    G = fa_split_chunks(S, nsplit)
    if workspace is None:
        ws_o = torch.empty((G, B, Hq, T, d), dtype=torch.float32, device=q.device)
        ws_lse = torch.empty((G, B, Hq, T), dtype=torch.float32, device=q.device)
    else:
        ws_o, ws_lse = workspace
        if (ws_o.dtype != torch.float32 or ws_lse.dtype != torch.float32 or not ws_o.is_contiguous()
                or not ws_lse.is_contiguous() or ws_o.numel() < G * B * Hq * T * d
                or ws_lse.numel() < G * B * Hq * T or ws_o.device != q.device or ws_lse.device != q.device):
            raise ValueError("workspace must be contiguous float32 tensors on the device of q, of at least "
                             "G*B*Hq*T*d and G*B*Hq*T elements")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_split(q, k, v, out, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, ws_o,
                          ws_lse, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_split")
    return out, lse
