"""Seeded synthetic inputs for the attention forward pass.

This module holds only input generation and the workload table: no step of
the attention method lives here.  Both the oracle side (tests, CPU baseline)
and the HIP side (tests, bench, smoke) draw their inputs from it, so that the
two see bit-identical tensors.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
``torch.randn`` in float32 for Q, then K, then V (in that order, each of shape
[B, H, N, d]); K is multiplied by ``k_mult`` in float32; each tensor is then
rounded to the workload dtype (bf16 by round-to-nearest-even).  The values are
i.i.d. N(0, 1), the distribution the attention pages' own examples use for
synthetic Q/K/V; ``k_mult = 3`` makes the softmax rows peaky.
"""

import math
from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_jump_qkv", "get", "hbm_once_bytes", "tile_stream_bytes"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    seed: int
    k_mult: float = 1.0
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d multiply-adds counted as 2 FLOPs each, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and O written once, plus the fp32 LSE."""
        elt = 2 if self.dtype == "bf16" else 4
        return 4 * self.B * self.H * self.N * self.d * elt + 4 * self.B * self.H * self.N


WORKLOADS = {
    "single_head_f32_n256_d64": Workload(
        "single_head_f32_n256_d64", 1, 1, 256, 64, "f32", False, 1,
        note="B=1 H=1 N=256 d=64 fp32, non-causal"),
    "ragged_n1000_d64_noncausal": Workload(
        "ragged_n1000_d64_noncausal", 4, 16, 1000, 64, "bf16", False, 2,
        note="B=4 H=16 N=1000 d=64 bf16, N not a tile multiple"),
    "ragged_n1000_d64_causal": Workload(
        "ragged_n1000_d64_causal", 4, 16, 1000, 64, "bf16", True, 2,
        note="B=4 H=16 N=1000 d=64 bf16 causal"),
    "n4096_d128_causal": Workload(
        "n4096_d128_causal", 2, 32, 4096, 128, "bf16", True, 3,
        note="B=2 H=32 N=4096 d=128 bf16 causal"),
    "n8192_d64_peaky": Workload(
        "n8192_d64_peaky", 8, 32, 8192, 64, "bf16", False, 4, k_mult=3.0,
        note="B=8 H=32 N=8192 d=64 bf16, K x3 (peaky rows), non-causal"),
    "longctx_n16384_d128_causal": Workload(
        "longctx_n16384_d128_causal", 1, 64, 16384, 128, "bf16", True, 5,
        note="B=1 H=64 N=16384 d=128 bf16 causal (headline workload)"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_qkv(B, H, N, d, dtype=torch.bfloat16, seed=0, k_mult=1.0):
    """Q, K, V as CPU tensors of ``dtype`` drawn per the module recipe."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    if k_mult != 1.0:
        k = k * float(k_mult)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def make_qkv_device(B, Hq, Hkv, T, S, d, dtype=torch.bfloat16, seed=0, device="cuda"):
    """Q [B, Hq, T, d], K and V [B, Hkv, S, d] drawn i.i.d. N(0, 1) directly
    in ``dtype`` on ``device`` by torch's generator for that device, seeded
    with ``seed`` (Q, then K, then V).  For inputs of billions of elements,
    which take too long to draw on the host; the tests copy the heads they
    check back to the host for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, T, d), generator=g, dtype=dtype, device=device)
    k = torch.randn((B, Hkv, S, d), generator=g, dtype=dtype, device=device)
    v = torch.randn((B, Hkv, S, d), generator=g, dtype=dtype, device=device)
    return q, k, v


def make_jump_qkv(B, Hq, Hkv, T, S, d, rows, key0, lift=60.0, seed=0, key1=None):
    """Q [B, Hq, T, d], K and V [B, Hkv, S, d] (bf16, CPU) in which only the
    chosen query rows see their scores jump.  Q, then K, then V are drawn
    i.i.d. N(0, 1) in float32 from a CPU generator seeded with ``seed``, then
    a unit vector u (a fourth draw, normalised) is projected out of every
    query and key row; each (head, row) pair in ``rows`` gets
    sqrt(lift * sqrt(d)) u added to its query, and every key from ``key0`` on
    (up to ``key1``, exclusive, when given) gets the same.  With the scale
    1/sqrt(d) the chosen rows' scores rise by ``lift`` nats on those keys;
    the other rows hold no component along u (up to the bf16 rounding)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, T, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    u = torch.randn(d, generator=g, dtype=torch.float32)
    u = u / u.norm()
    q = q - (q @ u)[..., None] * u
    k = k - (k @ u)[..., None] * u
    a = math.sqrt(lift * math.sqrt(d))
    for h, t in rows:
        q[:, h, t] += a * u
    k[:, :, key0:key1] += a * u
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def sample_rows(N, count, seed, include_ends=True):
    """Sorted distinct query rows: {0, N-1} plus random rows (seeded)."""
    import numpy as np
    rng = np.random.default_rng(int(seed))
    count = min(count, N)
    base = {0, N - 1} if include_ends else set()
    base = {r for r in base if 0 <= r < N}
    need = count - len(base)
    pool = np.setdiff1d(np.arange(N), np.array(sorted(base), dtype=np.int64))
    extra = rng.choice(pool, size=max(0, min(need, pool.size)), replace=False) if need > 0 else []
    return np.array(sorted(base | {int(x) for x in extra}), dtype=np.int64)


def sample_heads(B, H, count, seed):
    """Distinct (b, h) pairs chosen with a seeded generator, sorted."""
    import numpy as np
    rng = np.random.default_rng(int(seed) + 1000)
    count = min(count, B * H)
    flat = np.sort(rng.choice(B * H, size=count, replace=False))
    return [(int(f) // H, int(f) % H) for f in flat]


# ---------------------------------------------------------------- byte models
def hbm_once_bytes(B, H, N, d, elt=2):
    """Bytes a forward must move between HBM and the chip when every input
    row is read once and every output row written once: Q, K, V read, O
    written (elt bytes per element) and the fp32 LSE written.  The model of
    "FlashAttention V1" (infra.bea.ai), section "4. Memory Analysis", plus
    the LSE."""
    return 4 * B * H * N * d * elt + 4 * B * H * N


def tile_stream_bytes(B, H, N, d, Br, Bc, causal, elt=2):
    """Bytes the tiled forward requests from memory when nothing is reused
    across query tiles: Q once, every visible K and V tile once per query
    tile of Br rows, O and the fp32 LSE once.  The count of "Lecture 3 —
    FlashAttention-1 Algorithm" (jared-hpc.com), section "Why this is
    O(N^2 d^2 / M) bytes", with the causal loop bound (query tile i reads key
    tiles 0 .. ceil(min(N, (i+1) Br) / Bc) - 1)."""
    tr = -(-N // Br)
    tc = -(-N // Bc)
    kv_tiles = 0
    for i in range(tr):
        kv_tiles += -(-min(N, (i + 1) * Br) // Bc) if causal else tc
    per_head = N * d * elt + kv_tiles * 2 * Bc * d * elt + N * d * elt + 4 * N
    return B * H * per_head

