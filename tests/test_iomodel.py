"""The byte models used for IO validation, against their closed forms."""

import workloads


def test_read_once_is_eight_bytes_per_element_plus_lse():
    # "FlashAttention V1", "4. Memory Analysis": 4 x S x d_k x 2 bytes = 8 S d_k (bf16), plus fp32 LSE
    for (B, H, N, d) in [(1, 1, 4096, 128), (2, 3, 1000, 64)]:
        assert workloads.hbm_once_bytes(B, H, N, d) == B * H * (8 * N * d + 4 * N)


def test_tile_stream_kv_term_is_4_n2_d_over_br():
    # "Lecture 3", "Why this is O(N^2 d^2/M) bytes": KV traffic = 4 N^2 d / B_r bytes (bf16, divisible N)
    for (N, d, br, bc) in [(4096, 128, 256, 64), (8192, 64, 128, 128), (1024, 64, 64, 64)]:
        total = workloads.tile_stream_bytes(1, 1, N, d, br, bc, False)
        rest = 2 * N * d * 2 + 4 * N  # Q read, O written, LSE
        assert total - rest == 4 * N * N * d // br


def test_tile_stream_causal_bound():
    # query tile i reads key tiles 0 .. ceil((i+1) Br / Bc) - 1: with Br = r Bc that is
    # r (i + 1) tiles, r T_r (T_r + 1) / 2 in all
    N, d, br, bc = 4096, 128, 256, 64
    tr, r = N // br, br // bc
    kv = r * tr * (tr + 1) // 2 * 2 * bc * d * 2
    rest = 2 * N * d * 2 + 4 * N
    assert workloads.tile_stream_bytes(1, 1, N, d, br, bc, True) == kv + rest
    # ragged N: the last query tile's bound is ceil(N / Bc)
    n2 = 1000
    t = workloads.tile_stream_bytes(1, 1, n2, 64, 256, 128, True) - (2 * n2 * 64 * 2 + 4 * n2)
    tiles = sum(-(-min(n2, (i + 1) * 256) // 128) for i in range(-(-n2 // 256)))
    assert t == tiles * 2 * 128 * 64 * 2
