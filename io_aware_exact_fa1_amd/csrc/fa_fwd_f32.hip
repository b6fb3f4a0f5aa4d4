// fp32 attention forward for MI355X (gfx950): the kernel of fa_fwd_f32.
//
// What is computed is that of fa_fwd ("Lecture 3 - FlashAttention-1
// Algorithm" (jared-hpc.com), section "The forward loop (Algorithm 1 from
// the FA1 paper)"), for fp32 inputs in true fp32 arithmetic: fp32 products
// and sums on the vector ALUs, as "15. FlashAttention"
// (inference.shantanugoel.com), section "The kernel", keeps fp32 inputs in
// fp32 maths.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.h"
#include "fa_host.h"

namespace {

using namespace fa;

// fp32 path: true fp32 arithmetic on the vector ALUs.  A wave takes
// 64 / KL queries; the KL lanes of a query take every KL-th key of each
// LDS tile (lane kl: keys k0 + kl, k0 + kl + KL, ...) with their own online
// softmax state (m, l, acc), merged across the KL lanes at the end (the
// same log-sum-exp rule as a split over keys).  KL = 1 gives one query per
// thread (large problems, where K/V tiles are shared by 64 queries); KL = 16
// spreads small problems over 16 times more waves.
constexpr int F32_BK = 32;  // keys per LDS tile
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int D, bool CAUSAL, int KL>
__global__ void __launch_bounds__(64)
fa_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                  float* __restrict__ o, float* __restrict__ lse, int N, long long BH, float c) {
  constexpr int QW = 64 / KL;  // queries per wave
  // (b, h) from the y and z grid indices (each at most 65535)
  const long long bh = (long long)blockIdx.z * 65535 + blockIdx.y;
  if (bh >= BH) return;
  __shared__ float ks[F32_BK][D];
  __shared__ float vs[F32_BK][D];
  const int t = threadIdx.x;
  const int qi = t / KL, kl = t % KL;
  const int q0 = blockIdx.x * QW;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const int query = q0 + qi;
  const int qrow = min(query, N - 1);

  float qv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) qv[e] = q[hoff + (size_t)qrow * D + e];
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + QW) : N;
  for (int k0 = 0; k0 < kv_end; k0 += F32_BK) {
    // the tile's K and V rows as float4, every load of the tile issued
    // before the first is used
    constexpr int NL = F32_BK * D / 4 / 64;  // float4 per thread per matrix
    f32x4v kx[NL], vx[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = t + 64 * i;
      const int r = idx / (D / 4), e4 = idx % (D / 4);
      const size_t src = hoff + (size_t)min(k0 + r, N - 1) * D + 4 * e4;
      kx[i] = *(const f32x4v*)(k + src);
      vx[i] = *(const f32x4v*)(v + src);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = t + 64 * i;
      const int r = idx / (D / 4), e4 = idx % (D / 4);
      *(f32x4v*)&ks[r][4 * e4] = kx[i];
      *(f32x4v*)&vs[r][4 * e4] = vx[i];
    }
    __syncthreads();
    constexpr int NJ = F32_BK / KL;  // keys of this tile per lane
    float s[NJ];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = kl + KL * jj;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qv[e], ks[j][e], dot);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= query);
      s[jj] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m, mx);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - mref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const float p = (s[jj] == -INFINITY) ? 0.f : exp2f(s[jj] - mref);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vs[kl + KL * jj][e], acc[e]);
    }
    m = m_new;
  }
  // merge the KL lanes of each query (lanes kl = 0 .. KL-1 are adjacent)
  if (KL > 1) {
    float mq = m;
#pragma unroll
    for (int off = 1; off < KL; off *= 2) mq = fmaxf(mq, __shfl_xor(mq, off, 64));
    const float mref = (mq == -INFINITY) ? 0.f : mq;
    const float sc = exp2f(m - mref);  // 0 for a lane that saw no key
    l *= sc;
#pragma unroll
    for (int off = 1; off < KL; off *= 2) l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int e = 0; e < D; ++e) {
      float x = acc[e] * sc;
#pragma unroll
      for (int off = 1; off < KL; off *= 2) x += __shfl_xor(x, off, 64);
      acc[e] = x;
    }
    m = mq;
  }
  if (query < N && kl == 0) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) o[hoff + (size_t)query * D + e] = acc[e] * inv;
    lse[(size_t)bh * N + query] = (m + log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
void launch_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                float c, hipStream_t stream) {
  // fewer than 512 waves with one query per lane: spread each query over 16 lanes
  const long long bh = (long long)B * H;
  const unsigned gy = (unsigned)(bh < 65535 ? bh : 65535), gz = (unsigned)((bh + 65534) / 65535);
  if (bh * ((N + 63) / 64) < 512) {
    dim3 grid((N + 3) / 4, gy, gz);
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL, 16>), grid, dim3(64), 0, stream, q, k, v, o, lse, N, bh, c);
  } else {
    dim3 grid((N + 63) / 64, gy, gz);
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL, 1>), grid, dim3(64), 0, stream, q, k, v, o, lse, N, bh, c);
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
