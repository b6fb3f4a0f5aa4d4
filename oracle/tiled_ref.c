/* Exact attention by the tiled online-softmax recurrence, plain C, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the oracle's native twin of
 * oracle/tiled.py: a plain, slow CPU implementation that the tests check
 * against the oracle's pins and that bench.py times as a second CPU baseline.
 * Only tests/ and bench.py's cpu_baseline leg load it (through
 * oracle/native.py).  The HIP library never links, loads or calls it, and the
 * two share no code, header or constant.
 *
 * What it computes, per (batch, head), square self-attention:
 *   O = softmax(scale * Q K^T [causal: key j visible to query i iff j <= i]) V
 *   LSE_i = ln sum_j exp(scale * q_i . k_j)   (natural log, visible keys only)
 *
 * How (the pages' recurrence, in their order and notation):
 *   for each query tile of br rows:                       outer loop
 *     m = -inf, l = 0, acc = 0                            per row
 *     for each key tile of bc keys:                       inner loop
 *       s_j   = scale * q . k_j, or -inf when masked
 *       m_new = max(m, max_j s_j)
 *       ref   = m_new, or 0 while m_new = -inf           the safe reference
 *       alpha = exp(m - ref)                             rescales the old terms
 *       l     = alpha * l + sum_j exp(s_j - ref)
 *       acc   = alpha * acc + sum_j exp(s_j - ref) v_j
 *       m     = m_new
 *     O = acc / l, LSE = m + ln l                         written once
 *
 * Sources: "15. FlashAttention" (inference.shantanugoel.com), section "The
 * algorithm in plain PyTorch" (the same recurrence for one query and one head
 * in a native language; the safe reference of 0 for a row with no visible key
 * yet; a row that never sees a key is an error) and section "Online softmax:
 * normalize as you go" (the update of m, l, acc and O = acc / l).  "Lecture 3
 * - FlashAttention-1 Algorithm" (jared-hpc.com), section "The forward loop
 * (Algorithm 1 from the FA1 paper)": query tiles outside, key/value tiles
 * inside, O and LSE written once per query tile.
 */
#include <math.h>
#include <stdlib.h>

/* Status codes of fa_oracle_tiled_rows. */
#define ORACLE_OK 0
#define ORACLE_NO_VISIBLE_KEY (-1)
#define ORACLE_BAD_ARGS (-2)

/* Query rows [row0, row1) of one (batch, head).  q, k, v are n x d row-major
 * (query, key and value rows of this head), o is n x d and lse has n entries;
 * only rows row0 .. row1-1 of o and lse are written.  Query tiles of br rows
 * start at row0; key tiles of bc keys start at key 0.  Caller-owned memory
 * throughout; the function allocates only its own tile buffers. */
int fa_oracle_tiled_rows(const double* q, const double* k, const double* v, double* o, double* lse, long n,
                         long d, double scale, int causal, long br, long bc, long row0, long row1) {
  if (n < 1 || d < 1 || br < 1 || bc < 1 || row0 < 0 || row1 > n || row0 > row1) return ORACLE_BAD_ARGS;
  double* s = malloc(sizeof(double) * (size_t)bc);
  double* m = malloc(sizeof(double) * (size_t)br);
  double* l = malloc(sizeof(double) * (size_t)br);
  double* acc = malloc(sizeof(double) * (size_t)br * (size_t)d);
  if (!s || !m || !l || !acc) {
    free(s), free(m), free(l), free(acc);
    return ORACLE_BAD_ARGS;
  }
  int status = ORACLE_OK;
  for (long i0 = row0; i0 < row1 && status == ORACLE_OK; i0 += br) {
    const long i1 = i0 + br < row1 ? i0 + br : row1;
    for (long r = 0; r < i1 - i0; ++r) {
      m[r] = -INFINITY;
      l[r] = 0.0;
      for (long e = 0; e < d; ++e) acc[r * d + e] = 0.0;
    }
    for (long j0 = 0; j0 < n; j0 += bc) {
      const long j1 = j0 + bc < n ? j0 + bc : n;
      for (long i = i0; i < i1; ++i) {
        const long r = i - i0;
        /* scores of this row against the key tile, and their max */
        double mx = -INFINITY;
        for (long j = j0; j < j1; ++j) {
          double x = -INFINITY;
          if (!causal || j <= i) {
            x = 0.0;
            for (long e = 0; e < d; ++e) x += q[i * d + e] * k[j * d + e];
            x *= scale;
          }
          s[j - j0] = x;
          if (x > mx) mx = x;
        }
        const double m_new = m[r] > mx ? m[r] : mx;
        const double ref = m_new == -INFINITY ? 0.0 : m_new;
        const double alpha = exp(m[r] - ref);
        l[r] *= alpha;
        for (long e = 0; e < d; ++e) acc[r * d + e] *= alpha;
        for (long j = j0; j < j1; ++j) {
          const double p = exp(s[j - j0] - ref);
          l[r] += p;
          for (long e = 0; e < d; ++e) acc[r * d + e] += p * v[j * d + e];
        }
        m[r] = m_new;
      }
    }
    for (long i = i0; i < i1; ++i) {
      const long r = i - i0;
      if (!(l[r] > 0.0)) {
        status = ORACLE_NO_VISIBLE_KEY;
        break;
      }
      for (long e = 0; e < d; ++e) o[i * d + e] = acc[r * d + e] / l[r];
      lse[i] = m[r] + log(l[r]);
    }
  }
  free(s), free(m), free(l), free(acc);
  return status;
}
