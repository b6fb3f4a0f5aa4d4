// fp32 attention forward for MI355X (gfx950): the kernels of fa_fwd_f32.
//
// What is computed is that of fa_fwd ("Lecture 3 - FlashAttention-1
// Algorithm" (jared-hpc.com), section "The forward loop (Algorithm 1 from
// the FA1 paper)"), for fp32 inputs in true fp32 arithmetic: fp32 products
// and sums on the vector ALUs, as "15. FlashAttention"
// (inference.shantanugoel.com), section "The kernel", keeps fp32 inputs in
// fp32 maths.
//
// Two kernels:
//  * fa_fwd_f32_rows_kernel, for problems too small to fill the chip with
//    query tiles: a workgroup of 256 threads takes QB query rows and all
//    their keys at once, one key per thread per round of 256 keys, so that
//    a round costs one HBM/L2 round trip instead of a chain of dependent
//    small tiles;
//  * fa_fwd_f32_kernel otherwise: a wave streams 32-key K/V tiles through
//    LDS for its own 64 / DS query rows, DS lanes per row splitting the
//    head dimension (DS = 2 at d = 128 keeps a row's Q and accumulator in
//    128 registers per lane).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.h"
#include "fa_host.h"

namespace {

using namespace fa;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Small problems.  Workgroup = 4 waves = 256 threads, QB query rows
// [q0, q0 + QB) of one (b, h).  Keys go in rounds of 256: in round r,
// thread (w, lane) takes key 256 r + 64 w + lane.
//  1. The V rows of the round are copied HBM -> LDS (global_load_lds, no
//     register staging) while each thread loads its key's K row into
//     registers and forms its QB scores s = c * q . k (Q rows from LDS,
//     a broadcast read).
//  2. Each wave keeps its own online-softmax state per query row over the
//     keys it has seen (running max m, per-lane sums l, accumulator acc):
//     the wave max of the scores updates m, l and acc are rescaled by
//     exp2(m_old - m_new), p = exp2(s - m_new) goes to LDS.
//  3. P V over the wave's 64 keys of the round: lane owns output dims
//     lane + 64 i; weights and V rows are read from LDS.
// At the end the four waves' (m, l, acc) are merged with the log-sum-exp
// rule, O = sum_w e^{m_w - M} acc_w / sum_w e^{m_w - M} l_w,
// LSE = M + log2(L), converted to the natural log.
constexpr int kRowsKeys = 256;  // keys per round (one per thread)

template <int D, bool CAUSAL, int QB>
__global__ void __launch_bounds__(256)
fa_fwd_f32_rows_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                       float* __restrict__ o, float* __restrict__ lse, int N, long long BH, float c) {
  constexpr int DL = D / 64;  // output dims per lane in P V
  constexpr int C4 = D / 4;   // 16-byte chunks per row
  static_assert(4 * QB * D <= kRowsKeys * D, "merge buffer reuses the V buffer");
  // (b, h) from the y and z grid indices (each at most 65535)
  const long long bh = (long long)blockIdx.z * 65535 + blockIdx.y;
  if (bh >= BH) return;
  __shared__ __attribute__((aligned(1024))) float vs[kRowsKeys * D];  // V rows of the round
  __shared__ __attribute__((aligned(16))) float qs[QB * D];            // Q rows
  __shared__ __attribute__((aligned(16))) float ps[4 * 64 * QB];       // weights: [wave][key][query]
  __shared__ float mw[4 * QB], lw[4 * QB];                              // per-wave max and sum
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int q0 = blockIdx.x * QB;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const unsigned vbase = (unsigned)(uintptr_t)(float LDS_AS*)vs;

  for (int i = t; i < QB * C4; i += 256) {  // Q rows (rows past N clamped; never stored)
    const int r = i / C4, e4 = i % C4;
    ((f32x4v*)qs)[i] = *(const f32x4v*)(q + hoff + (size_t)min(q0 + r, N - 1) * D + 4 * e4);
  }
  __syncthreads();

  const int qlast = min(q0 + QB, N) - 1;  // last real query row of the block
  const int kv_end = CAUSAL ? qlast + 1 : N;
  const int rounds = (kv_end + kRowsKeys - 1) / kRowsKeys;
  float m[QB], ls[QB], acc[QB][DL];
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    m[qq] = -INFINITY;
    ls[qq] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DL; ++dd) acc[qq][dd] = 0.f;
  }

  for (int r = 0; r < rounds; ++r) {
    const int kbase = r * kRowsKeys;
    if (r > 0) __syncthreads();  // every wave is done reading the previous round's V rows
    // V rows kbase .. kbase + 255 (rows past N clamped to N - 1: finite,
    // weight 0): 16-byte chunk i = it * 256 + t of the round goes to LDS
    // byte 16 i, so a wave instruction fills 1 KiB at 16 (256 it + 64 w).
#pragma unroll 4
    for (int it = 0; it < C4; ++it) {
      const int idx = it * 256 + t;
      const int row = idx / C4, e4 = idx % C4;
      lds_copy16(v + hoff + (size_t)min(kbase + row, N - 1) * D + 4 * e4, vbase + 16u * (unsigned)(it * 256 + 64 * w));
    }
    // this thread's key row, then its scores
    const int key = kbase + 64 * w + lane;
    const f32x4v* krow = (const f32x4v*)(k + hoff + (size_t)min(key, N - 1) * D);
    f32x4v kr[C4];
#pragma unroll
    for (int e4 = 0; e4 < C4; ++e4) kr[e4] = krow[e4];
    float s[QB];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      float dot = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < C4; ++e4) {
        const f32x4v qv = ((const f32x4v*)qs)[qq * C4 + e4];
        dot = fmaf(qv.x, kr[e4].x, dot);
        dot = fmaf(qv.y, kr[e4].y, dot);
        dot = fmaf(qv.z, kr[e4].z, dot);
        dot = fmaf(qv.w, kr[e4].w, dot);
      }
      const bool vis = key < N && (!CAUSAL || key <= q0 + qq);
      s[qq] = vis ? dot * c : -INFINITY;
    }
    // online softmax of this wave's keys (the recurrence of "Lecture 3",
    // section "The forward loop", per wave)
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      const float m_new = fmaxf(m[qq], wave_max(s[qq]));
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;  // safe reference
      const float alpha = exp2f(m[qq] - mref);                // 0 while m = -inf
      const float p = exp2f(s[qq] - mref);                    // 0 for a masked key
      ls[qq] = ls[qq] * alpha + p;
#pragma unroll
      for (int dd = 0; dd < DL; ++dd) acc[qq][dd] *= alpha;
      m[qq] = m_new;
      ps[(w * 64 + lane) * QB + qq] = p;
    }
    wait_copies<0>();  // this thread's V copies (and K loads) have landed
    __syncthreads();   // ... and every thread's; the weights are visible
    // P V over keys kbase + 64 w .. + 63
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) {
      float pv[QB];
      if constexpr (QB == 2) {
        const f32x2v x = *(const f32x2v*)&ps[(w * 64 + kk) * QB];
        pv[0] = x.x;
        pv[1] = x.y;
      } else {
#pragma unroll
        for (int qq = 0; qq < QB; qq += 4) {
          const f32x4v x = *(const f32x4v*)&ps[(w * 64 + kk) * QB + qq];
          pv[qq] = x.x;
          pv[qq + 1] = x.y;
          pv[qq + 2] = x.z;
          pv[qq + 3] = x.w;
        }
      }
#pragma unroll
      for (int dd = 0; dd < DL; ++dd) {
        const float vv = vs[(64 * w + kk) * D + lane + 64 * dd];
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) acc[qq][dd] = fmaf(pv[qq], vv, acc[qq][dd]);
      }
    }
  }

  // merge the four waves (the accumulators go to the V buffer)
  __syncthreads();  // every wave is done with the V rows
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    const float lt = wave_sum(ls[qq]);
    if (lane == 0) {
      mw[w * QB + qq] = m[qq];
      lw[w * QB + qq] = lt;
    }
#pragma unroll
    for (int dd = 0; dd < DL; ++dd) vs[(w * QB + qq) * D + lane + 64 * dd] = acc[qq][dd];
  }
  __syncthreads();
  for (int i = t; i < QB * D; i += 256) {
    const int qq = i / D, e = i % D;
    if (q0 + qq >= N) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mw[ww * QB + qq]);
    float L = 0.f, x = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float sc = exp2f(mw[ww * QB + qq] - M);  // 0 for a wave that saw no key
      L = fmaf(sc, lw[ww * QB + qq], L);
      x = fmaf(sc, vs[(ww * QB + qq) * D + e], x);
    }
    o[hoff + (size_t)(q0 + qq) * D + e] = x / L;
    if (e == 0) lse[(size_t)bh * N + q0 + qq] = (M + log2f(L)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Larger problems: a wave takes 64 / DS query rows; the DS lanes of a row
// hold D / DS of its dimensions (Q and acc), form partial dot products that
// one lane swap completes, and update their dimensions of acc.  K/V tiles of
// 32 keys are copied HBM -> LDS (global_load_lds, every copy of a tile in
// flight at once, no register staging) and the running max rescales l and
// acc on every tile.
constexpr int F32_BK = 32;  // keys per LDS tile

template <int D, bool CAUSAL, int DS>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
fa_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                  float* __restrict__ o, float* __restrict__ lse, int N, long long BH, float c) {
  constexpr int QW = 64 / DS;  // queries per wave
  constexpr int DL = D / DS;   // dimensions per lane
  constexpr int NL = F32_BK * D / 4 / 64;  // 16-byte copies per lane per matrix and tile
  const long long bh = (long long)blockIdx.z * 65535 + blockIdx.y;
  if (bh >= BH) return;
  __shared__ __attribute__((aligned(1024))) float ks[F32_BK * D];
  __shared__ __attribute__((aligned(1024))) float vs[F32_BK * D];
  const unsigned kbase = (unsigned)(uintptr_t)(float LDS_AS*)ks;
  const unsigned vbase = (unsigned)(uintptr_t)(float LDS_AS*)vs;
  const int t = threadIdx.x;
  const int qi = t / DS, ds = t % DS;
  const int q0 = blockIdx.x * QW;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const int query = q0 + qi;
  const int qrow = min(query, N - 1);
  const int dbase = ds * DL;

  float qv[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) qv[e] = q[hoff + (size_t)qrow * D + dbase + e];
  float acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + QW) : N;
  for (int k0 = 0; k0 < kv_end; k0 += F32_BK) {
    __syncthreads();  // the previous tile's reads are done
    // 16-byte chunk idx = t + 64 i of the tile: row idx / (D/4), to LDS
    // byte 16 idx (rows past N clamped to N - 1: finite, weight 0)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = t + 64 * i;
      const int r = idx / (D / 4), e4 = idx % (D / 4);
      const size_t src = hoff + (size_t)min(k0 + r, N - 1) * D + 4 * e4;
      lds_copy16(k + src, kbase + 1024u * i);
      lds_copy16(v + src, vbase + 1024u * i);
    }
    wait_copies<0>();
    __syncthreads();
    float s[F32_BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < F32_BK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) dot = fmaf(qv[e], ks[j * D + dbase + e], dot);
      if (DS > 1) dot += __shfl_xor(dot, 1, 64);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= query);
      s[j] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - mref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < F32_BK; ++j) {
      const float p = (s[j] == -INFINITY) ? 0.f : exp2f(s[j] - mref);
      l += p;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = fmaf(p, vs[j * D + dbase + e], acc[e]);
    }
    m = m_new;
  }
  if (query < N) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[hoff + (size_t)query * D + dbase + e] = acc[e] * inv;
    if (ds == 0) lse[(size_t)bh * N + query] = (m + log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
void launch_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                float c, hipStream_t stream) {
  const long long bh = (long long)B * H;
  const unsigned gy = (unsigned)(bh < 65535 ? bh : 65535), gz = (unsigned)((bh + 65534) / 65535);
  constexpr int DS = D / 64;
  const long long waves = bh * ((N + 64 / DS - 1) / (64 / DS));
  if (waves < 512) {
    // too few query tiles to fill the chip: whole rows of keys per round
    if (bh * N <= 1024) {
      dim3 grid((N + 1) / 2, gy, gz);
      hipLaunchKernelGGL((fa_fwd_f32_rows_kernel<D, CAUSAL, 2>), grid, dim3(256), 0, stream, q, k, v, o, lse, N,
                         bh, c);
    } else {
      dim3 grid((N + 7) / 8, gy, gz);
      hipLaunchKernelGGL((fa_fwd_f32_rows_kernel<D, CAUSAL, 8>), grid, dim3(256), 0, stream, q, k, v, o, lse, N,
                         bh, c);
    }
  } else {
    dim3 grid((N + 64 / DS - 1) / (64 / DS), gy, gz);
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL, DS>), grid, dim3(64), 0, stream, q, k, v, o, lse, N, bh, c);
  }
}

}  // namespace

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                          int N, int d, float scale, int causal, hipStream_t stream) {
  const int st = host_check(q, k, v, o, lse, B, H, N, d, scale, 4);
  if (st != FA_OK) return st;
  if ((long long)B * H * N == 0) return FA_OK;
  const float c = scale * kLog2e;
  if (d == 128) {
    if (causal) launch_f32<128, true>(q, k, v, o, lse, B, H, N, c, stream);
    else launch_f32<128, false>(q, k, v, o, lse, B, H, N, c, stream);
  } else {
    if (causal) launch_f32<64, true>(q, k, v, o, lse, B, H, N, c, stream);
    else launch_f32<64, false>(q, k, v, o, lse, B, H, N, c, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
