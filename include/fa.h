/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The library computes, for every (batch b, head h), the exact attention
 * forward pass over square self-attention inputs:
 *
 *     O   = softmax(scale * Q K^T [+ causal mask]) V
 *     LSE = row-wise logsumexp(scale * Q K^T [+ causal mask])   (natural log)
 *
 * without ever forming the N x N score matrix in memory: Q is split into
 * row tiles, every K/V tile streams through on-chip LDS, and a running row
 * max m and sum-exp l (online softmax) rescale the partial output, which is
 * written to HBM once as O = a / l together with LSE = m + ln l.
 *
 * Definitions followed:
 *   - Problem statement (Q, K, V in, O out, O = softmax(QK^T / sqrt d) V):
 *     "FlashAttention V1" (infra.bea.ai), section "3. The Algorithm";
 *     "15. FlashAttention" (inference.shantanugoel.com), section "The score
 *     matrix is the problem".
 *   - The LSE output, m + log(l) per query row, written with O:
 *     "Lecture 3 - FlashAttention-1 Algorithm" (jared-hpc.com), section
 *     "The forward loop"; the logsumexp reading of it: "FlashAttention：从
 *     IO-Aware Attention 到 GPU Work Partitioning" (blog.euler0525.cn),
 *     section "减少 Non-Matmul FLOPs".
 *   - Causal rule (key j visible to query i iff j <= i) and the masked,
 *     never-read tail of N not a multiple of the tile: "15. FlashAttention",
 *     section "The kernel".
 *   - fp32 inputs computed in true fp32, not a reduced-precision matrix
 *     mode: "15. FlashAttention", section "The kernel" (the input_precision
 *     note).
 *
 * Layout (all entry points): Q, K, V and O are dense, contiguous, row-major
 * [B, H, N, d] arrays; element (b, h, n, e) sits at ((b*H + h)*N + n)*d + e.
 * LSE is a dense fp32 [B, H, N] array.  All pointers are DEVICE pointers
 * (memory of the current HIP device).
 *
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 * frees nothing and keeps no pointer after the call returns.  O and LSE are
 * written in full; they must not overlap Q, K, V or each other.
 *
 * Streams: work is enqueued on `stream` (0 = the null stream) and the call
 * returns without synchronising; the caller synchronises.
 *
 * Errors: every entry point returns FA_OK (0) or one of the FA_ERR_* codes
 * below.  Argument errors are detected on the host before any launch, and
 * then nothing is enqueued and nothing is written.  B*H*N == 0 is a no-op
 * that returns FA_OK.  FA_ERR_LAUNCH reports the HIP error of the launch
 * (from hipGetLastError, which may also carry an earlier, unrelated error of
 * the calling thread).
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a null pointer while B*H*N > 0                 */
    FA_ERR_SHAPE = 2,     /* B, H or N negative, or sizes overflow the grid */
    FA_ERR_HEAD_DIM = 3,  /* d not in {64, 128}                             */
    FA_ERR_SCALE = 4,     /* scale is NaN or infinite                       */
    FA_ERR_ALIAS = 5,     /* O or LSE overlaps Q, K, V or each other        */
    FA_ERR_LAUNCH = 6,    /* the HIP launch reported an error               */
    FA_ERR_ALIGN = 7,     /* a pointer is not aligned to 16 bytes           */
    FA_ERR_VARIANT = 8,   /* fa_fwd_ex/_split: Hq % Hkv, S == 0, offset, window, nsplit */
    FA_ERR_SCRATCH = 9    /* fa_fwd_split_noalloc: partials exceed FA_SPLIT_NOALLOC_BYTES */
};

/*
 * Exact attention forward, bf16 inputs and output, fp32 statistics.
 *
 *   q, k, v : const bf16 [B, H, N, d] device arrays (bf16 = IEEE binary32
 *             with the low 16 bits dropped), 16-byte aligned.
 *   o       : bf16 [B, H, N, d] device array, written: O rounded to bf16
 *             with round-to-nearest-even.
 *   lse     : float [B, H, N] device array, written: natural-log logsumexp
 *             of the scaled, masked scores of each query row.
 *   B, H, N : batch, heads, sequence length (N >= 1 when B*H > 0; any N,
 *             tiles need not divide it).
 *   d       : head dimension, 64 or 128.
 *   scale   : finite multiplier of Q K^T (usually 1/sqrt(d)); any sign.
 *   causal  : 0 = no mask; nonzero = key j is visible to query i iff j <= i.
 *   stream  : HIP stream to enqueue on.
 *
 * Arithmetic: Q K^T and P V run on bf16 matrix cores with fp32 accumulation;
 * the row max, the exponentials (base 2 with log2(e) folded into the scale),
 * the row sums, the running output and LSE are fp32; P is rounded to bf16
 * only as the operand of P V, while l sums the unrounded values and gives
 * LSE.  O is divided by the sum of the rounded weights P V multiplied: l
 * plus, on the tiles whose weights dominate a row, the difference between
 * the rounded and the unrounded weights ("15. FlashAttention", section "The
 * kernel": fp32 statistics, p cast to the value type for P V).  The
 * exponent reference of a row is the max of its first key tile with a
 * visible key (any common reference gives the same O and LSE in exact
 * arithmetic); on a tile where
 * a row's weights would outgrow it by more than 2^16, that row takes the
 * running-max step of the recurrence ("15. FlashAttention", section "Online
 * softmax: normalize as you go": new reference, l and the accumulator
 * rescaled by exp(m_old - m_new)), so no weight exceeds 2^16.
 * Range: the fp32 accumulator then holds at most N * 2^16 * max|V|, so the
 * results are those of the recurrence while N * max|V| stays below about
 * 2^112 (the recurrence's own fp32 accumulator needs N * max|V| below
 * about 2^128); beyond that, O may overflow to inf.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Exact attention forward for fp32 inputs and output, computed in true fp32
 * (fp32 products and sums on the vector ALUs; no reduced-precision matrix
 * mode).  Arguments, layout, errors and semantics as fa_fwd, with q, k, v
 * and o fp32 [B, H, N, d] device arrays (16-byte aligned).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

/*
 * Whether the forward entry points take head dimension d with element type
 * dtype (FA_DTYPE_BF16: fa_fwd, fa_fwd_ex, fa_fwd_split, fa_bwd;
 * FA_DTYPE_F32: fa_fwd_f32): 1 if so, 0 if not (any other d or dtype).
 * A pure host query; no HIP call.  The head dimensions are those of the
 * pages' kernels ("15. FlashAttention", section "The kernel": the head
 * dimension is a compile-time block size; "FlashAttention V1", section "4.
 * Memory Analysis": d = 64 and 128 are the sizes analysed).
 */
#define FA_DTYPE_BF16 0
#define FA_DTYPE_F32 1
int fa_supported(int d, int dtype);

/*
 * Host-side argument check of fa_fwd / fa_fwd_f32 without any HIP call:
 * returns the status those entry points would return before launching.
 * elem_bytes is 2 (bf16) or 4 (fp32).  Lets tests and callers validate on
 * machines without a GPU.
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int B, int H, int N, int d, float scale, int causal, int elem_bytes);

/*
 * Variants of fa_fwd (bf16): grouped K/V heads (GQA), queries at an offset
 * into a longer key sequence (chunked prefill, decode), a sliding window.
 *
 * What is computed, following "15. FlashAttention"
 * (inference.shantanugoel.com), section "The kernel": query head h of
 * batch b reads K/V head h / (Hq / Hkv); query row i sits at absolute
 * position offset + i; key j is visible to row i iff j < S and, when causal,
 * j <= offset + i and, with a window W > 0, j >= offset + i - W + 1 (the
 * window covers W keys ending at the query's own position; it requires the
 * causal mask).  Then O = softmax(scale * q k^T over the visible keys) v and
 * LSE = logsumexp of those scores, per row.
 *
 * Arguments:
 *   q, o   bf16 [B, Hq, T, d] contiguous device memory (q read, o written).
 *   k, v   bf16 [B, Hkv, S, d] contiguous device memory, read only.
 *   lse    fp32 [B, Hq, T], natural log, written.
 *   offset position of query row 0 (causal only; ignored otherwise), with
 *          0 <= offset <= S - T so that no row is empty; S - T is the usual
 *          choice (the queries are the newest positions).
 *   window 0 for none, else W >= 1 (causal only).
 *   B, d, scale, causal, stream: as for fa_fwd.
 * Errors as for fa_fwd, plus FA_ERR_VARIANT for Hq % Hkv != 0, S == 0, an
 * offset outside [0, S - T] or a window without the causal mask.  With
 * Hq == Hkv, T == S, offset 0 and no window the result equals fa_fwd's bit
 * for bit (the same kernel, with the variants' index arithmetic).
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int T,
              int S, int d, float scale, int causal, int offset, int window, hipStream_t stream);

/* Host-side argument check of fa_fwd_ex without any HIP call. */
int fa_check_args_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
                     int Hkv, int T, int S, int d, float scale, int causal, int offset, int window);

/*
 * Split-KV form of fa_fwd_ex (flash-decoding): the keys are cut into G
 * chunks, each (query tile, chunk) pair is its own work unit, and a second
 * kernel merges the partial results.  For short query sequences (decode:
 * T = 1) this gives the GPU B * Hq * G work units instead of B * Hq.
 *
 * What is computed, following "15. FlashAttention"
 * (inference.shantanugoel.com), section "Decode is different:
 * flash-decoding": chunk g holds keys [g * C, (g + 1) * C); for each query
 * row it yields the softmax output O_g over that chunk's visible keys and
 * their log-sum-exp L_g (O_g = 0, L_g = -inf where the row sees none of
 * them); then L = log sum_g exp(L_g) and O = sum_g exp(L_g - L) O_g.  The
 * result is the same attention as fa_fwd_ex (equal up to rounding order).
 *
 * Arguments:
 *   q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window,
 *          stream: as for fa_fwd_ex (o and lse receive the merged result).
 *   nsplit requested number of chunks, 1 <= nsplit <= 4096.  The chunk
 *          length is C = ceil(ceil(S / nsplit) / 128) * 128 keys (whole
 *          key tiles) and the number of chunks used is G = ceil(S / C) =
 *          fa_split_chunks(S, nsplit) <= nsplit.
 *   ws_o   fp32 [G, B, Hq, T, d] workspace (device memory, 16-byte
 *          aligned), owned by the caller; on return it holds the partials
 *          O_g.
 *   ws_lse fp32 [G, B, Hq, T] workspace (device memory), owned by the
 *          caller; on return it holds L_g.
 * Two kernels serve this.  With at most 32 query rows per K/V head
 * ((Hq / Hkv) * T <= 32: decode, short chunked prefill) a small-tile kernel
 * runs one workgroup per (batch, K/V head, chunk), the query heads of the
 * group times the T rows forming the 32 columns of its matrix products, so
 * that each K/V byte is read once; with one chunk it writes O and LSE
 * itself.  Otherwise each (256-row query tile, chunk) is a work unit of
 * the fa_fwd_ex kernel, and with one chunk the call is fa_fwd_ex itself.
 * When G == 1 the workspaces are neither used nor checked (they may be
 * NULL).
 * Errors as for fa_fwd_ex, plus FA_ERR_VARIANT for nsplit outside
 * [1, 4096], FA_ERR_NULL / FA_ERR_ALIGN for a missing or misaligned
 * workspace, FA_ERR_ALIAS when a workspace overlaps an input, an output
 * or the other workspace, and FA_ERR_SHAPE when a launch would exceed
 * 2^32 work items.  The kernels run in order on `stream` (the partial
 * kernel, then for G > 1 the merge); nothing is allocated, no memset is
 * issued and no atomics are used, so results are deterministic and the
 * call can be captured in a HIP graph.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int T,
                 int S, int d, float scale, int causal, int offset, int window, int nsplit, float* ws_o,
                 float* ws_lse, hipStream_t stream);

/*
 * fa_fwd_split for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving (decode) loops, harnesses that forbid
 * hipMalloc.  Same arguments, result and errors as fa_fwd_split without
 * ws_o / ws_lse: the partials go to a device array the library holds,
 * FA_SPLIT_NOALLOC_BYTES bytes per device, held from the first call on a
 * device (which looks up its address) until the process ends.  Nothing is
 * allocated, freed or memset by the call.
 *   Limit: G * B * Hq * T * (d + 1) * 4 <= FA_SPLIT_NOALLOC_BYTES, with
 *   G = fa_split_chunks(S, nsplit) (a single chunk uses no scratch);
 *   larger calls return FA_ERR_SCRATCH before any launch.
 *   Sharing: every call on one device uses the same array, which keeps the
 *   last call's partials; calls that overlap in time on one device (two
 *   streams, two threads) race on it and must be serialised by the caller.
 * FA_ERR_LAUNCH also reports a failure to find the array's device address.
 */
#define FA_SPLIT_NOALLOC_BYTES (32u << 20)
int fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int T, int S, int d, float scale, int causal, int offset, int window, int nsplit,
                         hipStream_t stream);

/* Number of key chunks G that fa_fwd_split uses for S keys and a requested
 * nsplit (1 for S <= 0 or nsplit < 1); sizes its workspaces. */
int fa_split_chunks(int S, int nsplit);

/* Host-side argument check of fa_fwd_split without any HIP call. */
int fa_check_args_split(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                        int Hq, int Hkv, int T, int S, int d, float scale, int causal, int offset, int window,
                        int nsplit, const float* ws_o, const float* ws_lse);

/*
 * Backward pass of fa_fwd (bf16): the gradients dQ, dK, dV of sum(O * dO)
 * with respect to Q, K, V, recomputed from Q, K, V and the forward's LSE
 * instead of a stored probability matrix.
 *
 * What is computed, per (b, h), following "FlashAttention：从 IO-Aware
 * Attention 到 GPU Work Partitioning" (blog.euler0525.cn), sections
 * "Tiling、Fusion 与 Backward Recomputation" and "减少 Non-Matmul FLOPs", and
 * "FlashAttention V1" (infra.bea.ai), section "5. The Backward Pass":
 *   P  = exp(scale * Q K^T - LSE)   (causal: 0 where key > query)
 *   D_i = O_i . dO_i
 *   dS = P * (dO V^T - D)
 *   dV = P^T dO,  dQ = scale * dS K,  dK = scale * dS^T Q
 * (the pages write the gradients for unscaled scores; the scale of the
 * forward enters dQ and dK once by the chain rule).
 *
 * Arguments:
 *   q, k, v, o, dout  bf16 [B, H, N, d] contiguous, device memory, read only:
 *                     the forward's inputs and output (O as fa_fwd wrote
 *                     it) and the upstream gradient dO.
 *   lse               fp32 [B, H, N], the natural-log LSE fa_fwd wrote.
 *   dq, dk, dv        bf16 [B, H, N, d], written entirely (outputs).
 *   delta             fp32 [B, H, N] workspace owned by the caller; on
 *                     return it holds D_i = O_i . dO_i.
 *   B, H, N, d, scale, causal, stream: as for fa_fwd (scale and causal must
 *                     be those of the forward call).
 * Layout, ownership, stream semantics and error codes as for fa_fwd; in
 * addition dq, dk, dv and delta must not overlap each other or any input
 * (FA_ERR_ALIAS).  The two kernels run in order on `stream`; nothing is
 * allocated and no atomics are used, so results are deterministic.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream);

/*
 * Host-side argument check of fa_bwd without any HIP call: returns the
 * status fa_bwd would return before launching.
 */
int fa_bwd_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const void* dq, const void* dk, const void* dv, const float* delta,
                      int B, int H, int N, int d, float scale, int causal);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
