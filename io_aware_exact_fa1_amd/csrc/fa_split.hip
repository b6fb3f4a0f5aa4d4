// Split-KV attention forward (flash-decoding) for MI355X (gfx950): the
// small-tile partial kernel, the merge kernel and the C entry points
// fa_fwd_split, fa_fwd_split_noalloc, fa_check_args_split and
// fa_split_chunks.
//
// What is computed: "15. FlashAttention" (inference.shantanugoel.com),
// section "Decode is different: flash-decoding": the keys are cut into
// chunks, each chunk yields per query row the softmax output over its
// visible keys and their log-sum-exp, and the partials are merged by the
// log-sum-exp rule.  The masks, grouped K/V heads, query offset and window
// are those of fa_fwd_ex (same page, section "The kernel").

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_host.h"

// Scratch of fa_fwd_split_noalloc: the fp32 partials of a call (ws_o, then
// ws_lse).  Every device the library runs on holds its own copy until the
// process ends; all calls on a device share it.  In host code `scratch` is
// only a handle: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[FA_SPLIT_NOALLOC_BYTES];

namespace {

using namespace fa;

// Split-KV merge ("15. FlashAttention", section "Decode is different:
// flash-decoding"): per row, L = log sum_g exp(L_g) and
// O = sum_g exp(L_g - L) O_g over the G partials (a partial with
// L_g = -inf, a chunk the row sees no key of, has weight 0).  A workgroup
// of 256 threads takes RB rows; within a row, thread (gi, col) takes four
// output dims (col) of the partials g = gi, gi + NGL, ..., so that the
// partial rows are read in parallel (coalesced float4) rather than one
// after another, and the NGL partial sums are added in LDS.  NGL is the
// largest power of two <= min(G, 256 / (D/4)) and RB = 256 / (D/4) / NGL.
inline int merge_ngl(int D, int G) {
  int n = 1;
  while (2 * n <= G && 2 * n <= 256 / (D / 4)) n *= 2;
  return n;
}

inline dim3 merge_grid(long long rows, int D, int G) {
  const long long rb = 256 / (D / 4) / merge_ngl(D, G);
  const long long blocks = (rows + rb - 1) / rb;
  return dim3((unsigned)(blocks < 65536 ? blocks : 65536), (unsigned)((blocks + 65535) / 65536));
}

template <int D>
__global__ void __launch_bounds__(256)
fa_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, uint16_t* __restrict__ o,
                float* __restrict__ lse, long long rows, int nsplit, int ngl) {
  constexpr int NC = D / 4;       // float4 columns per row
  constexpr int NS = 256 / NC;    // (row, gi) slots per workgroup
  __shared__ float smax[NS];
  __shared__ float stot[NS];
  __shared__ __attribute__((aligned(16))) float sacc[NS][D];
  const int col = threadIdx.x % NC;
  const int slot = threadIdx.x / NC;           // rl * ngl + gi
  const int gi = slot % ngl, rl = slot / ngl;  // (ngl is a power of two)
  const int rb = NS / ngl;
  // (a 2-D grid: 65536 workgroups per grid row)
  const long long row = ((long long)blockIdx.y * 65536 + blockIdx.x) * rb + rl;
  const bool live = row < rows;
  float mx = -INFINITY;
  if (live) {
#pragma unroll 4
    for (int g = gi; g < nsplit; g += ngl) mx = fmaxf(mx, ws_lse[(long long)g * rows + row]);
  }
  if (col == 0) smax[slot] = mx;
  __syncthreads();
  mx = -INFINITY;
  for (int j = 0; j < ngl; ++j) mx = fmaxf(mx, smax[rl * ngl + j]);
  // (mx is finite for a live row: every row sees a key of some chunk)
  float tot = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (live) {
#pragma unroll 4
    for (int g = gi; g < nsplit; g += ngl) {
      const float lg = ws_lse[(long long)g * rows + row];
      const float4 x = *(const float4*)(ws_o + ((long long)g * rows + row) * D + 4 * col);
      const float wgt = lg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lg - mx) * kLog2e);
      tot += wgt;
      a0 = fmaf(wgt, x.x, a0);
      a1 = fmaf(wgt, x.y, a1);
      a2 = fmaf(wgt, x.z, a2);
      a3 = fmaf(wgt, x.w, a3);
    }
  }
  if (col == 0) stot[slot] = tot;
  sacc[slot][4 * col + 0] = a0;
  sacc[slot][4 * col + 1] = a1;
  sacc[slot][4 * col + 2] = a2;
  sacc[slot][4 * col + 3] = a3;
  __syncthreads();
  if (gi != 0 || !live) return;
  tot = 0.f;
  a0 = a1 = a2 = a3 = 0.f;
  for (int j = 0; j < ngl; ++j) {
    const int sl = rl * ngl + j;
    tot += stot[sl];
    a0 += sacc[sl][4 * col + 0];
    a1 += sacc[sl][4 * col + 1];
    a2 += sacc[sl][4 * col + 2];
    a3 += sacc[sl][4 * col + 3];
  }
  const float inv = 1.f / tot;
  bf16x4 ov;
  ov[0] = (__bf16)(a0 * inv);
  ov[1] = (__bf16)(a1 * inv);
  ov[2] = (__bf16)(a2 * inv);
  ov[3] = (__bf16)(a3 * inv);
  *(u32x2*)(o + row * D + 4 * col) = __builtin_bit_cast(u32x2, ov);
  if (col == 0) lse[row] = mx + __logf(tot);
}

template <int D>
void launch_merge(float* ws_o, float* ws_lse, void* o, float* lse, long long rows, int G, hipStream_t stream) {
  hipLaunchKernelGGL(fa_merge_kernel<D>, merge_grid(rows, D, G), dim3(256), 0, stream, ws_o, ws_lse, (uint16_t*)o,
                     lse, rows, G, merge_ngl(D, G));
}

// ---------------------------------------------------------------------------
// Split-KV with few query rows per K/V head (decode, short chunked prefill):
// "15. FlashAttention", section "Decode is different: flash-decoding".
// A work unit is (batch b, K/V head hk, key chunk g).  The R = group * T
// query rows that read K/V head hk (the group's query heads times the T
// rows) are the 32 columns of the matrix products (columns past R repeat
// row R-1 and are discarded), so each K/V byte of the chunk is read once
// for all of them.  The DEC_NW waves of the workgroup take turns over the
// chunk's 32-key tiles (wave w: tiles w, w + DEC_NW, ...); each wave
// streams its own tiles through a private two-stage LDS ring (copy of the
// next tile in flight while the current one is computed, no workgroup
// barrier), keeps an exact online softmax (running max, rescale of l and
// acc on every tile), and at the end the waves' (m, l, acc) are combined
// in LDS.  G = 1 writes O (bf16) and LSE directly; G > 1 writes the fp32
// partial (O_g, L_g) of the chunk for fa_merge_kernel, with O_g = 0,
// L_g = -inf for a row that sees no key of the chunk.
typedef float f32x4d __attribute__((ext_vector_type(4)));
constexpr int DEC_NW = 4;   // waves per workgroup
constexpr int DEC_KT = 32;  // keys per wave tile

template <int D>
struct DecCfg {
  static constexpr int ROWB = D * 2;        // bytes of one K/V row
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per 1 KB wave-wide copy
  static constexpr int TB = DEC_KT * ROWB;  // bytes of one K (or V) tile
  static constexpr int NCP = TB / 1024;     // copies per matrix per tile
  static constexpr int NG = 16 / RPI;       // copies per swizzle period (16 rows)
  static constexpr int STB = 2 * TB;        // one stage: the K tile, then the V tile
  static constexpr int WB = 2 * STB;        // one wave's ring of two stages
  static constexpr int KB = D / 16;         // 16-deep k-steps of K Q^T
  static constexpr int DB = D / 32;         // 32-dim output blocks
  static constexpr int OSTR = D + 4;        // row stride (floats) of the combine buffer
  static_assert(NCP % NG == 0 && 2 * NCP < 64, "copies per tile");
  static_assert(DEC_NW * WB <= 160 * 1024, "LDS size");
  static_assert(DEC_NW * (32 * OSTR + 64) * 4 <= DEC_NW * WB, "the combine buffer fits in the rings");
};

struct DecArgs {
  int B, Hq, Hkv, T, S, offset, window, chunk, G, R;
  long long rows;  // B * Hq * T
  float c;         // |scale| * log2(e)
  unsigned qsign;  // sign flip of Q for a negative scale
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(DEC_NW * 64)
fa_decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                 uint16_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ ws_o,
                 float* __restrict__ ws_lse, DecArgs a) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DEC_NW * C::WB];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int u = blockIdx.x;  // ((b * Hkv) + hk) * G + g
  const int g = u % a.G;
  const int bk = u / a.G;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int group = a.Hq / a.Hkv;

  // this lane's query column: row r -> query head hk * group + r / T, row r % T
  const int r = min(l32, a.R - 1);
  const int t = r % a.T;
  const size_t qrow = ((size_t)b * a.Hq + (size_t)(hk * group + r / a.T)) * a.T + t;
  bf16x8 qr[C::KB];
  {
    const uint16_t* src = q + qrow * D + 8 * h;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      u32x4 x = *(const u32x4*)(src + 16 * kb);
      x ^= a.qsign;
      qr[kb] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.S * D;
  const uint16_t* kh = k + kvoff;
  const uint16_t* vh = v + kvoff;

  // keys of this unit: the chunk, clipped to what some row can see
  int k_lo = g * a.chunk;
  int k_hi = min(a.S, (g + 1) * a.chunk);
  if (CAUSAL) {
    k_hi = min(k_hi, a.offset + a.T);  // the last row sits at offset + T - 1
    if (a.window > 0) k_lo = max(k_lo, a.offset - a.window + 1);
  }
  const int t_lo = k_lo / DEC_KT;
  const int ntile = k_hi > k_lo ? (k_hi + DEC_KT - 1) / DEC_KT - t_lo : 0;
  const int nmine = __builtin_amdgcn_readfirstlane(ntile > w ? (ntile - w + DEC_NW - 1) / DEC_NW : 0);

  // this lane's visible keys: lo <= key <= hi
  const int hi = CAUSAL ? min(a.offset + t, a.S - 1) : a.S - 1;
  const int lo = (CAUSAL && a.window > 0) ? a.offset + t - a.window + 1 : 0;

  // LDS offsets within a stage (swizzled as in the main kernel)
  const unsigned wbase = (unsigned)(uintptr_t)(const unsigned char LDS_AS*)smem + (unsigned)w * C::WB;
  int lok[C::KB];
  {
    const int kf = swz<D>(l32);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) lok[kb] = l32 * C::ROWB + 16 * ((2 * kb + h) ^ kf);
  }
  int lov[C::DB][2];
  {
    const int vr = 4 * h + ((lane >> 2) & 3);
    const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int vf0 = swz<D>(vr), vf1 = swz<D>(vr + 8);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int dim = 32 * db + vdim;
      lov[db][0] = C::TB + vr * C::ROWB + 16 * ((dim >> 3) ^ vf0) + 2 * (dim & 7);
      lov[db][1] = C::TB + (vr + 8) * C::ROWB + 16 * ((dim >> 3) ^ vf1) + 2 * (dim & 7);
    }
  }
  // copies: copy ii of a tile moves rows RPI*ii .. RPI*ii + RPI-1; lane
  // offsets repeat every NG copies (the swizzle period)
  unsigned gofs[C::NG];
#pragma unroll
  for (int j = 0; j < C::NG; ++j) {
    const int row = C::RPI * j + lane / C::CPR;
    gofs[j] = (unsigned)((lane / C::CPR) * C::ROWB + ((lane % C::CPR) ^ swz<D>(row)) * 16);
  }
  auto copy_tile = [&](const uint16_t* src, int k0, unsigned dst) __attribute__((always_inline)) {
    if (k0 + DEC_KT <= a.S) {
#pragma unroll
      for (int ii = 0; ii < C::NCP; ++ii)
        lds_copy16_s((const char*)src + ((size_t)k0 + (size_t)(C::RPI * ii)) * C::ROWB, gofs[ii % C::NG],
                     dst + ii * 1024);
    } else {  // the sequence's last tile: rows past S - 1 repeat row S - 1 (masked)
#pragma unroll
      for (int ii = 0; ii < C::NCP; ++ii) {
        const int row = C::RPI * ii + lane / C::CPR;
        const int chunk = (lane % C::CPR) ^ swz<D>(row);
        lds_copy16(src + (size_t)min(k0 + row, a.S - 1) * D + (size_t)chunk * 8, dst + ii * 1024);
      }
    }
  };
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int k0 = __builtin_amdgcn_readfirstlane((t_lo + w + DEC_NW * i) * DEC_KT);
    const unsigned st = wbase + (unsigned)(i & 1) * C::STB;
    copy_tile(kh, k0, st);
    copy_tile(vh, k0, st + C::TB);
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
  const f32x16 zero = {};

  if (nmine > 0) issue(0);
  for (int i = 0; i < nmine; ++i) {
    if (i + 1 < nmine) {
      issue(i + 1);
      wait_copies<2 * C::NCP>();  // tile i has landed, tile i + 1 in flight
    } else {
      wait_copies<0>();
    }
    // no LDS read of the tile moves above the wait
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const unsigned st = wbase + (unsigned)(i & 1) * C::STB;
    const int k0 = (t_lo + w + DEC_NW * i) * DEC_KT;
    // S^T = K Q^T: register j holds key k0 + 8*(j/4) + 4h + j%4
    f32x16 s = zero;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      const bf16x8 kk = *(const bf16x8 LDS_AS*)(lds + st + lok[kb]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[kb], s, 0, 0, 0);
    }
    // mask, exact online softmax
    const int rhi = hi - (k0 + 4 * h), rlo = lo - (k0 + 4 * h);
    float mq = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int rel = 8 * (j >> 2) + (j & 3);
      s[j] = (rel <= rhi && rel >= rlo) ? s[j] : -INFINITY;
      mq = __builtin_fmaxf(mq, s[j]);
    }
    const float mx = half_max(mq);
    const float mxs = (mx == -INFINITY) ? -INFINITY : mx * a.c;
    const float m_new = __builtin_fmaxf(m, mxs);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);  // 0 while m = -inf
    m = m_new;
    float ts = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], a.c, -mref));
      ts += s[j];
    }
    lsum = fmaf(lsum, alpha, ts);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[db][j] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[kb2][j] = (__bf16)s[8 * kb2 + j];
    // acc += V^T P^T (V^T through LDS transpose reads, keys in the order of pb)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int off = (int)st + kb2 * 16 * C::ROWB;
        const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + off + lov[db][0]));
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + off + lov[db][1]));
        const bf16x8 va = __builtin_shufflevector(__builtin_bit_cast(bf16x4, x0), __builtin_bit_cast(bf16x4, x1),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb2], acc[db], 0, 0, 0);
      }
  }
  const float lt = half_sum(lsum);

  // combine the waves: acc [NW][32][OSTR], then m [NW][32], l [NW][32]
  __syncthreads();  // every wave is done with its ring
  float LDS_AS* cb = (float LDS_AS*)smem;
  float LDS_AS* cm = cb + DEC_NW * 32 * C::OSTR;
  float LDS_AS* cl = cm + DEC_NW * 32;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x4d x = {acc[db][4 * a4 + 0], acc[db][4 * a4 + 1], acc[db][4 * a4 + 2], acc[db][4 * a4 + 3]};
      *(f32x4d LDS_AS*)(cb + (w * 32 + l32) * C::OSTR + 32 * db + 8 * a4 + 4 * h) = x;
    }
  if (h == 0) {
    cm[w * 32 + l32] = m;
    cl[w * 32 + l32] = lt;
  }
  __syncthreads();
  constexpr int Q4 = D / 4;  // float4 columns per row
#pragma unroll
  for (int it = threadIdx.x; it < 32 * Q4; it += DEC_NW * 64) {
    const int row = it / Q4, col = it % Q4;
    if (row >= a.R) continue;
    float mw[DEC_NW];
    float mmax = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < DEC_NW; ++ww) {
      mw[ww] = cm[ww * 32 + row];
      mmax = __builtin_fmaxf(mmax, mw[ww]);
    }
    float tot = 0.f;
    float4 ov = {0.f, 0.f, 0.f, 0.f};
    if (mmax != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < DEC_NW; ++ww) {
        const float e = __builtin_amdgcn_exp2f(mw[ww] - mmax);  // 0 for a wave that saw no key
        const f32x4d x = *(const f32x4d LDS_AS*)(cb + (ww * 32 + row) * C::OSTR + 4 * col);
        tot = fmaf(e, cl[ww * 32 + row], tot);
        ov.x = fmaf(e, x[0], ov.x);
        ov.y = fmaf(e, x[1], ov.y);
        ov.z = fmaf(e, x[2], ov.z);
        ov.w = fmaf(e, x[3], ov.w);
      }
    }
    const bool empty = !(tot > 0.f);
    const float inv = empty ? 0.f : 1.f / tot;
    const float L = empty ? -INFINITY : (mmax + __log2f(tot)) * kLn2;
    const size_t orow = ((size_t)b * a.Hq + (size_t)(hk * group + row / a.T)) * a.T + row % a.T;
    if (a.G == 1) {
      bf16x4 ob;
      ob[0] = (__bf16)(ov.x * inv);
      ob[1] = (__bf16)(ov.y * inv);
      ob[2] = (__bf16)(ov.z * inv);
      ob[3] = (__bf16)(ov.w * inv);
      *(u32x2*)(o + orow * D + 4 * col) = __builtin_bit_cast(u32x2, ob);
      if (col == 0) lse[orow] = L;
    } else {
      const size_t prow = (size_t)g * (size_t)a.rows + orow;
      float4 x;
      x.x = ov.x * inv;
      x.y = ov.y * inv;
      x.z = ov.z * inv;
      x.w = ov.w * inv;
      *(float4*)(ws_o + prow * D + 4 * col) = x;
      if (col == 0) ws_lse[prow] = L;
    }
  }
}

template <int D, bool CAUSAL>
void launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* ws_o, float* ws_lse,
                   const DecArgs& a, hipStream_t stream) {
  const long long units = (long long)a.B * a.Hkv * a.G;
  hipLaunchKernelGGL((fa_decode_kernel<D, CAUSAL>), dim3((unsigned)units), dim3(DEC_NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, ws_o, ws_lse, a);
}

}  // namespace

// Key chunk of each split: whole 128-key tiles (a multiple of both key tile
// widths), so that no tile straddles two chunks.
static int split_chunk(int S, int nsplit) { return ((S + nsplit - 1) / nsplit + 127) / 128 * 128; }

extern "C" int fa_split_chunks(int S, int nsplit) {
  if (S <= 0 || nsplit < 1) return 1;
  const int chunk = split_chunk(S, nsplit);
  return (S + chunk - 1) / chunk;
}

extern "C" int fa_check_args_split(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                   int B, int Hq, int Hkv, int T, int S, int d, float scale, int causal,
                                   int offset, int window, int nsplit, const float* ws_o, const float* ws_lse) {
  const int st = host_check_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window);
  if (st != FA_OK) return st;
  if (nsplit < 1 || nsplit > 4096) return FA_ERR_VARIANT;
  const long long rows = (long long)B * Hq * T;
  if (rows == 0) return FA_OK;
  const int g = fa_split_chunks(S, nsplit);
  // the launches must fit the 32-bit work-item count of a dispatch
  const bool small = (long long)(Hq / Hkv) * T <= 32;
  const long long items = small ? (long long)B * Hkv * g * (DEC_NW * 64)
                                : (long long)B * Hq * ((T + 255) / 256) * g * 512;
  if ((small || g > 1) && (items > 0xFFFFFFFFLL || rows > 65535LL * 65536)) return FA_ERR_SHAPE;
  if (g == 1) return FA_OK;  // no workspace used
  if (!ws_o || !ws_lse) return FA_ERR_NULL;
  if (((uintptr_t)ws_o & 15) || ((uintptr_t)ws_lse & 3)) return FA_ERR_ALIGN;
  if ((long long)B * Hq * ((T + 31) / 32) * g > (1LL << 30)) return FA_ERR_SHAPE;
  const size_t wob = (size_t)g * rows * d * 4, wlb = (size_t)g * rows * 4;
  const size_t qb = (size_t)rows * d * 2, kb = (size_t)B * Hkv * S * d * 2, lb = (size_t)rows * 4;
  const void* all[5] = {q, k, v, o, lse};
  const size_t sz[5] = {qb, kb, kb, qb, lb};
  for (int i = 0; i < 5; ++i)
    if (host_overlaps(ws_o, wob, all[i], sz[i]) || host_overlaps(ws_lse, wlb, all[i], sz[i])) return FA_ERR_ALIAS;
  if (host_overlaps(ws_o, wob, ws_lse, wlb)) return FA_ERR_ALIAS;
  return FA_OK;
}

namespace {

// Device address of the scratch on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int T, int S, int d, float scale, int causal, int offset, int window,
                            int nsplit, float* ws_o, float* ws_lse, hipStream_t stream) {
  const int st = fa_check_args_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit,
                                     ws_o, ws_lse);
  if (st != FA_OK) return st;
  const long long rows = (long long)B * Hq * T;
  if (rows == 0) return FA_OK;
  const int g = fa_split_chunks(S, nsplit);
  const int chunk = split_chunk(S, nsplit);
  const unsigned qsign = (scale < 0.f) ? 0x80008000u : 0u;  // as in fa_fwd
  const float c = scale == 0.f ? 0x1p-100f : fabsf(scale) * kLog2e;
  const int off = causal ? offset : 0;
  const int wnd = causal ? window : 0;
  if ((long long)(Hq / Hkv) * T <= 32) {
    // few query rows per K/V head: the small-tile kernel (writes O and LSE
    // itself when there is one chunk)
    const DecArgs da{B, Hq, Hkv, T, S, off, wnd, chunk, g, (Hq / Hkv) * T, rows, c, qsign};
    if (d == 128) {
      if (causal) launch_decode<128, true>(q, k, v, o, lse, ws_o, ws_lse, da, stream);
      else launch_decode<128, false>(q, k, v, o, lse, ws_o, ws_lse, da, stream);
    } else {
      if (causal) launch_decode<64, true>(q, k, v, o, lse, ws_o, ws_lse, da, stream);
      else launch_decode<64, false>(q, k, v, o, lse, ws_o, ws_lse, da, stream);
    }
    if (g > 1) {
      if (d == 128)
        launch_merge<128>(ws_o, ws_lse, o, lse, rows, g, stream);
      else
        launch_merge<64>(ws_o, ws_lse, o, lse, rows, g, stream);
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  }
  if (g == 1)  // one chunk: the direct path
    return fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, stream);
  host_launch_ex_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, causal, off, wnd, c, qsign, g, chunk, ws_o, ws_lse,
                       stream);
  if (d == 128) launch_merge<128>(ws_o, ws_lse, o, lse, rows, g, stream);
  else launch_merge<64>(ws_o, ws_lse, o, lse, rows, g, stream);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                    int Hq, int Hkv, int T, int S, int d, float scale, int causal, int offset,
                                    int window, int nsplit, hipStream_t stream) {
  const int st = host_check_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window);
  if (st != FA_OK) return st;
  if (nsplit < 1 || nsplit > 4096) return FA_ERR_VARIANT;
  const long long rows = (long long)B * Hq * T;
  if (rows == 0) return FA_OK;
  const int g = fa_split_chunks(S, nsplit);
  float* ws_o = nullptr;
  float* ws_lse = nullptr;
  if (g > 1) {
    // ws_o [G, B, Hq, T, d] then ws_lse [G, B, Hq, T], fp32 (rows <= 2^40,
    // G <= 4096, d + 1 <= 129: the product fits 64 bits)
    const unsigned long long need = (unsigned long long)g * (unsigned long long)rows * (unsigned)(d + 1) * 4ull;
    if (need > (unsigned long long)FA_SPLIT_NOALLOC_BYTES) return FA_ERR_SCRATCH;
    void* p = nullptr;
    const int sst = device_scratch(&p);
    if (sst != FA_OK) return sst;
    ws_o = (float*)p;
    ws_lse = ws_o + (size_t)g * (size_t)rows * d;
  }
  // the same checks and kernels as fa_fwd_split, on the scratch (every
  // partial the merge reads is written first by the partial kernel, so
  // nothing needs clearing between calls)
  return fa_fwd_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, ws_o, ws_lse,
                      stream);
}
