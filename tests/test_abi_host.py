"""Host-side checks of the C-ABI library (no GPU needed, no kernel launch).

The library must load, export every entry point ``include/fa.h`` declares,
and reject bad arguments on the host before any HIP call.
"""

import ctypes
import math
import os
import re

import pytest

import io_aware_exact_fa1_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(["fa_bwd", "fa_bwd_check_args", "fa_check_args", "fa_check_args_ex",
                                           "fa_check_args_split", "fa_fwd", "fa_fwd_ex", "fa_fwd_f32",
                                           "fa_fwd_split", "fa_fwd_split_noalloc", "fa_split_chunks",
                                           "fa_strerror", "fa_supported"])


def test_binding_exports_match_the_header():
    assert sorted(fa.EXPORTED) == declared_functions()


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    raw = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value, name


def test_supported_head_dims_and_types():
    for dtype in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32):
        assert fa.fa_supported(64, dtype) == 1
        assert fa.fa_supported(128, dtype) == 1
        for d in (0, 1, 32, 63, 65, 96, 127, 129, 256, -64):
            assert fa.fa_supported(d, dtype) == 0, (d, dtype)
    for dtype in (-1, 2, 3, 99):
        assert fa.fa_supported(128, dtype) == 0
    # the checks agree: a supported head dimension passes, any other is FA_ERR_HEAD_DIM
    for d in (32, 64, 96, 128, 256):
        st = fa.fa_check_args(Q, K, V, O, L, 1, 1, 8, d, 0.125, 0, 2)
        assert (st == fa.FA_OK) == bool(fa.fa_supported(d, fa.FA_DTYPE_BF16)), d
        if st != fa.FA_OK:
            assert st == fa.FA_ERR_HEAD_DIM


def test_strerror_covers_codes():
    for code in range(0, 10):
        s = fa.fa_strerror(code)
        assert s and s != "unknown status", code
    assert fa.fa_strerror(99) == "unknown status"


# Fake device addresses: aligned, disjoint, never dereferenced (argument checks
# return before any HIP call).
Q, K, V, O, L = (0x10000000 * (i + 1) for i in range(5))


@pytest.mark.parametrize("elem", [2, 4])
def test_check_args_ok(elem):
    assert fa.fa_check_args(Q, K, V, O, L, 2, 3, 100, 64, 0.125, 1, elem) == fa.FA_OK
    assert fa.fa_check_args(Q, K, V, O, L, 1, 1, 1, 128, -2.0, 0, elem) == fa.FA_OK


@pytest.mark.parametrize("args,code", [
    ((Q, K, V, O, L, -1, 1, 8, 64, 1.0, 0), fa.FA_ERR_SHAPE),
    ((Q, K, V, O, L, 1, -1, 8, 64, 1.0, 0), fa.FA_ERR_SHAPE),
    ((Q, K, V, O, L, 1, 1, -8, 64, 1.0, 0), fa.FA_ERR_SHAPE),
    ((Q, K, V, O, L, 1, 1, 8, 32, 1.0, 0), fa.FA_ERR_HEAD_DIM),
    ((Q, K, V, O, L, 1, 1, 8, 96, 1.0, 0), fa.FA_ERR_HEAD_DIM),
    ((Q, K, V, O, L, 1, 1, 8, 64, math.nan, 0), fa.FA_ERR_SCALE),
    ((Q, K, V, O, L, 1, 1, 8, 64, math.inf, 0), fa.FA_ERR_SCALE),
    ((None, K, V, O, L, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_NULL),
    ((Q, K, V, O, None, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_NULL),
    ((Q + 8, K, V, O, L, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_ALIGN),
    ((Q, K, V, O, L + 2, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_ALIGN),
    ((Q, K, V, Q, L, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_ALIAS),
    ((Q, K, V, O, O + 64, 1, 1, 8, 64, 1.0, 0), fa.FA_ERR_ALIAS),
    ((Q, K, V, O, L, 1 << 20, 1 << 20, 8, 64, 1.0, 0), fa.FA_ERR_SHAPE),
])
def test_check_args_errors(args, code):
    assert fa.fa_check_args(*args, 2) == code


def test_entry_points_reject_bad_args_before_any_launch():
    # These return on the host before touching HIP, so they are safe without a GPU.
    assert fa.fa_fwd(Q, K, V, O, L, 1, 1, 8, 80, 1.0, 0, 0) == fa.FA_ERR_HEAD_DIM
    assert fa.fa_fwd_f32(Q, K, V, O, L, 1, 1, 8, 64, math.nan, 0, 0) == fa.FA_ERR_SCALE
    assert fa.fa_fwd(None, K, V, O, L, 1, 1, 8, 64, 1.0, 0, 0) == fa.FA_ERR_NULL


def test_empty_problem_is_a_noop():
    # B*H*N == 0: FA_OK with no launch, even with null pointers.
    assert fa.fa_fwd(None, None, None, None, None, 0, 4, 16, 64, 1.0, 1, 0) == fa.FA_OK
    assert fa.fa_fwd_f32(None, None, None, None, None, 2, 4, 0, 128, 1.0, 0, 0) == fa.FA_OK


def test_forward_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)


# backward: fake addresses of o, dout, dq, dk, dv, delta
DO, DQ, DK, DV, DL = (0x10000000 * (i + 6) for i in range(5))


def _bwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2, N=40, d=64,
             scale=0.125, causal=1)
    a.update(kw)
    return fa.fa_bwd_check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                                a["delta"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"])


def test_bwd_check_args_ok():
    assert _bwd() == fa.FA_OK
    assert _bwd(d=128, causal=0, scale=-1.0) == fa.FA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_HEAD_DIM),
    (dict(scale=math.inf), fa.FA_ERR_SCALE),
    (dict(dout=None), fa.FA_ERR_NULL),
    (dict(delta=None), fa.FA_ERR_NULL),
    (dict(dq=DQ + 8), fa.FA_ERR_ALIGN),
    (dict(delta=DL + 2), fa.FA_ERR_ALIGN),
    (dict(dq=Q), fa.FA_ERR_ALIAS),          # output over an input
    (dict(dv=DK), fa.FA_ERR_ALIAS),         # two outputs overlap
    (dict(delta=L), fa.FA_ERR_ALIAS),       # workspace over the forward's LSE
    (dict(delta=DQ + 64), fa.FA_ERR_ALIAS),
])
def test_bwd_check_args_errors(kw, code):
    assert _bwd(**kw) == code


def test_bwd_rejects_and_noops_on_the_host():
    assert fa.fa_bwd(Q, K, V, O, L, DO, DQ, DK, DV, DL, 1, 1, 8, 96, 1.0, 0, 0) == fa.FA_ERR_HEAD_DIM
    assert fa.fa_bwd(*([None] * 10), 0, 3, 16, 64, 1.0, 1, 0) == fa.FA_OK


def test_backward_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.backward(x, x, x, x, lse, x)


def _ex(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=8, Hkv=2, T=100, S=400, d=128, scale=0.1, causal=1, offset=300,
             window=0)
    a.update(kw)
    return fa.fa_check_args_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"], a["S"],
                               a["d"], a["scale"], a["causal"], a["offset"], a["window"])


def test_ex_check_args_ok():
    assert _ex() == fa.FA_OK
    assert _ex(window=64) == fa.FA_OK
    assert _ex(causal=0, offset=-5, T=1000, S=3) == fa.FA_OK   # cross-attention: offset ignored
    assert _ex(T=1, offset=399) == fa.FA_OK                    # decode
    assert _ex(B=0, q=None) == fa.FA_OK                        # empty


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=3), fa.FA_ERR_VARIANT),            # 8 query heads over 3 KV heads
    (dict(Hkv=0), fa.FA_ERR_VARIANT),
    (dict(S=0), fa.FA_ERR_VARIANT),
    (dict(offset=301), fa.FA_ERR_VARIANT),       # > S - T
    (dict(offset=-1), fa.FA_ERR_VARIANT),
    (dict(T=500, offset=0), fa.FA_ERR_VARIANT),  # T > S with the causal mask
    (dict(window=-1), fa.FA_ERR_VARIANT),
    (dict(window=8, causal=0), fa.FA_ERR_VARIANT),
    (dict(d=96), fa.FA_ERR_HEAD_DIM),
    (dict(T=-1), fa.FA_ERR_SHAPE),
    (dict(k=None), fa.FA_ERR_NULL),
    (dict(o=K), fa.FA_ERR_ALIAS),
    (dict(lse=O + 128), fa.FA_ERR_ALIAS),
])
def test_ex_check_args_errors(kw, code):
    assert _ex(**kw) == code


WO, WL = 0x60000000, 0x70000000


def _split(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=8, Hkv=2, T=1, S=4000, d=128, scale=0.1, causal=1, offset=3999,
             window=0, nsplit=8, ws_o=WO, ws_lse=WL)
    a.update(kw)
    return fa.fa_check_args_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"],
                                  a["S"], a["d"], a["scale"], a["causal"], a["offset"], a["window"], a["nsplit"],
                                  a["ws_o"], a["ws_lse"])


@pytest.mark.parametrize("S,nsplit,G", [
    (1, 1, 1), (1, 8, 1), (128, 2, 1), (129, 2, 2), (300, 4, 3), (4000, 8, 8), (16384, 8, 8), (16384, 3, 3),
    (16384, 4096, 128), (1000, 1000, 8), (0, 4, 1), (100, 0, 1),
])
def test_split_chunks(S, nsplit, G):
    """G = ceil(S / C) with C = ceil(ceil(S / nsplit) / 128) * 128: whole
    128-key chunks, never more than nsplit of them."""
    assert fa.fa_split_chunks(S, nsplit) == G
    if S > 0 and nsplit > 0:
        C = -(-(-(-S // nsplit)) // 128) * 128
        assert G == -(-S // C) and G <= nsplit and (G - 1) * C < S <= G * C


def test_split_check_args_ok():
    assert _split() == fa.FA_OK
    assert _split(nsplit=1, ws_o=None, ws_lse=None) == fa.FA_OK     # one chunk: no workspace
    assert _split(S=100, offset=99, ws_o=None, ws_lse=None) == fa.FA_OK
    assert _split(T=100, offset=0, window=300) == fa.FA_OK
    assert _split(causal=0, T=7) == fa.FA_OK
    assert _split(B=0, q=None, ws_o=None) == fa.FA_OK                  # empty


@pytest.mark.parametrize("kw,code", [
    (dict(nsplit=0), fa.FA_ERR_VARIANT),
    (dict(nsplit=4097), fa.FA_ERR_VARIANT),
    (dict(ws_o=None), fa.FA_ERR_NULL),
    (dict(ws_lse=None), fa.FA_ERR_NULL),
    (dict(ws_o=WO + 8), fa.FA_ERR_ALIGN),
    (dict(ws_lse=WL + 2), fa.FA_ERR_ALIGN),
    (dict(ws_o=K), fa.FA_ERR_ALIAS),
    (dict(ws_lse=O), fa.FA_ERR_ALIAS),
    (dict(ws_lse=WO + 64), fa.FA_ERR_ALIAS),
    (dict(Hkv=3), fa.FA_ERR_VARIANT),             # the fa_fwd_ex checks come first
    (dict(d=80), fa.FA_ERR_HEAD_DIM),
])
def test_split_check_args_errors(kw, code):
    assert _split(**kw) == code


def test_split_rejects_on_the_host():
    assert fa.fa_fwd_split(Q, K, V, O, L, 1, 2, 2, 1, 1000, 128, 0.1, 1, 999, 0, 0, WO, WL, 0) == fa.FA_ERR_VARIANT
    assert fa.fa_fwd_split(Q, K, V, O, L, 1, 2, 2, 1, 1000, 128, 0.1, 1, 999, 0, 4, None, WL, 0) == fa.FA_ERR_NULL
    assert fa.fa_fwd_split(None, None, None, None, None, 0, 2, 2, 1, 1000, 128, 0.1, 1, 999, 0, 4, None, None,
                           0) == fa.FA_OK


def test_split_rejects_launches_past_32_bit_work_items():
    """4096 x 64 K/V heads in 64 chunks: 2^24 small-tile workgroups of 256
    work items do not fit one dispatch."""
    P = [(i + 1) << 44 for i in range(7)]
    st = fa.fa_check_args_split(P[0], P[1], P[2], P[3], P[4], 4096, 64, 64, 1, 8192, 128, 0.1, 1, 8191, 0, 64,
                                P[5], P[6])
    assert st == fa.FA_ERR_SHAPE
    st = fa.fa_check_args_split(P[0], P[1], P[2], P[3], P[4], 4096, 64, 64, 1, 8192, 128, 0.1, 1, 8191, 0, 32,
                                P[5], P[6])
    assert st == fa.FA_OK


def test_split_noalloc_rejects_on_the_host():
    """The argument checks of fa_fwd_split, then the scratch limit: partials
    of G * B * Hq * T * (d + 1) * 4 bytes beyond FA_SPLIT_NOALLOC_BYTES are
    refused before any HIP call."""
    text = open(HEADER).read()
    assert re.search(r"#define FA_SPLIT_NOALLOC_BYTES \(32u << 20\)", text)
    assert fa.FA_SPLIT_NOALLOC_BYTES == 32 << 20
    call = fa.fa_fwd_split_noalloc
    assert call(Q, K, V, O, L, 1, 2, 2, 1, 1000, 128, 0.1, 1, 999, 0, 0, 0) == fa.FA_ERR_VARIANT    # nsplit
    assert call(Q, K, V, O, L, 1, 3, 2, 1, 1000, 128, 0.1, 1, 999, 0, 4, 0) == fa.FA_ERR_VARIANT    # Hq % Hkv
    assert call(Q, K, V, O, L, 1, 2, 2, 1, 1000, 80, 0.1, 1, 999, 0, 4, 0) == fa.FA_ERR_HEAD_DIM
    assert call(None, None, None, None, None, 0, 2, 2, 1, 1000, 128, 0.1, 1, 999, 0, 4, 0) == fa.FA_OK
    # 64 query heads x 4096 rows in 4 chunks of d = 128: 4 * 64 * 4096 * 129 * 4 bytes = 541 MB
    P = [(i + 1) << 44 for i in range(5)]
    assert call(P[0], P[1], P[2], P[3], P[4], 1, 64, 64, 4096, 4096, 128, 0.1, 1, 0, 0, 4, 0) == fa.FA_ERR_SCRATCH
    # the largest decode that fits: G * rows * (d + 1) * 4 <= 32 MiB
    G, d = 32, 128
    rows = (32 << 20) // (G * (d + 1) * 4)
    assert call(P[0], P[1], P[2], P[3], P[4], 1, rows + 1, 1, 1, 32 * 128, d, 0.1, 1, 32 * 128 - 1, 0, G,
                0) == fa.FA_ERR_SCRATCH

