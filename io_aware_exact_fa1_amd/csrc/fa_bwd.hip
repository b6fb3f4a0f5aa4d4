// Exact attention backward for MI355X (gfx950, CDNA4): HIP kernels + C ABI.
//
// What is computed (per batch b, head h; square self-attention), from the
// forward's inputs, its output O, its row log-sum-exp L and an upstream
// gradient dO:
//   P  = exp(scale * Q K^T - L)          [causal: 0 where key > query]
//   D_i = O_i . dO_i
//   dS = P * (dO V^T - D)
//   dV = P^T dO,   dQ = scale * dS K,   dK = scale * dS^T Q
// Sources: "FlashAttention：从 IO-Aware Attention 到 GPU Work Partitioning"
// (blog.euler0525.cn), section "Tiling、Fusion 与 Backward Recomputation"
// (the gradient formulas, D_i = O_i . dO_i, recomputing S and P instead of
// storing P) and section "减少 Non-Matmul FLOPs" (P rebuilt from the saved
// log-sum-exp); "FlashAttention V1" (infra.bea.ai), section "5. The Backward
// Pass"; "Lecture 3 — FlashAttention-1 Algorithm" (jared-hpc.com), section
// "Backward in one sentence".  The pages write the gradients for unscaled
// scores; with S = scale * Q K^T the chain rule puts the factor scale on dQ
// and dK.
//
// gfx950 design: two kernels, no atomics, nothing allocated.
//  * dQ kernel (query-tiled, like the forward): a workgroup owns 128 query
//    rows (4 waves x 32) and streams 32-key tiles of K and V through LDS.
//    Per tile: S^T = K Q^T and dP^T = V dO^T on the matrix cores (one query
//    per lane, Q and dO in registers), P and dS^T in registers, then
//    dQ^T += K^T dS^T with K^T read from the LDS tile by transpose reads and
//    dS^T (bf16) as the register operand.  It also forms D_i = O_i . dO_i
//    for its rows and writes D to the caller's workspace.
//  * dK/dV kernel (key-tiled): a workgroup owns 128 keys (4 waves x 32; K
//    rows in registers, V rows resident in LDS, so that two workgroups fit
//    on a CU) and streams 32-query tiles of Q, dO and their L and D through
//    LDS.  Per tile: S = Q K^T and dP = dO V^T with one key
//    per lane, P and dS in registers, then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read by transpose reads.
//  Both use the LDS swizzle and the operand layouts of the forward kernel,
//  and copy tiles HBM -> LDS with global_load_lds, double-buffered.  With a
//  causal mask the tiles above the diagonal are skipped and work units pair
//  a heavy tile with a light one.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

using namespace fa;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DQ_NST = 4;  // LDS stages of the dQ kernel's K/V ring

// Tile configuration of both backward kernels.
template <int D_>
struct BCfg {
  static constexpr int D = D_;
  static constexpr int ROWB = D * 2;        // bytes of one bf16 row
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per 1 KB wave-wide copy
  static constexpr int KB = D / 16;         // 16-deep k-steps over d
  static constexpr int DB = D / 32;         // 32-wide blocks of d
  static constexpr int NW = 4;              // waves per workgroup
  static constexpr int ROWS = 32 * NW;      // rows a workgroup owns
  static constexpr int T = 32;              // rows of a streamed tile
  static constexpr int TB = T * ROWB;       // bytes of one streamed tile of one matrix
  static constexpr int NINST = TB / 1024;   // 1 KB copies per matrix per tile
  static constexpr int NI = NINST / NW;     // ... per wave
  static constexpr int XB = 1024;           // room for the L and D rows of a query tile (256 B)
  static constexpr int STAGE = 2 * TB + XB; // one LDS stage: two matrices (+ L, D)
  static constexpr int DQSTAGE = 2 * TB;    // one stage of the dQ kernel: K and V
  static_assert(NINST % NW == 0 && NI >= 1, "copies must split evenly over the waves");
  static_assert((NW * RPI) % 16 == 0, "a wave's copy rows must be a swizzle period apart");
};

// Per-lane LDS offsets within a streamed tile (bytes from the tile start).
template <class C>
struct BLane {
  int row[C::KB];     // row operand: tile row l%32, dims 16kb + 8(l/32) .. +7
  int tr[C::DB][2];   // transposed operand of dim block db: rows +0 / +8
  unsigned g;         // copies: this lane's 16 bytes within a 1 KB block
};

template <class C>
__device__ __forceinline__ void blane(BLane<C>& bl, int w, int lane) {
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int f = swz<C::D>(l32);
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) bl.row[kb] = l32 * C::ROWB + 16 * ((2 * kb + h) ^ f);
  // transpose reads: lane (g = l/16, r, b) reads tile row 4h + r [+8], dims
  // 32*db + 16*(g%2) + 4b .. +3; afterwards lane l holds
  // tile[16*kq + 4h + 0..3 (+8)][32*db + l%32] for the 16-row block kq.
  const int vr = 4 * h + ((lane >> 2) & 3);
  const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int f0 = swz<C::D>(vr), f1 = swz<C::D>(vr + 8);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int dim = 32 * db + vdim;
    bl.tr[db][0] = vr * C::ROWB + 16 * ((dim >> 3) ^ f0) + 2 * (dim & 7);
    bl.tr[db][1] = (vr + 8) * C::ROWB + 16 * ((dim >> 3) ^ f1) + 2 * (dim & 7);
  }
  const int row = w * C::RPI + lane / C::CPR;
  const int chunk = (lane % C::CPR) ^ swz<C::D>(row);
  bl.g = (unsigned)(lane / C::CPR * C::ROWB + chunk * 16);
}

// This wave's share of the HBM -> LDS copy of rows r0 .. r0+T-1 of one
// [N, D] matrix into the tile at LDS address dst.  Rows past N - 1 are
// clamped to row N - 1 (never read past the array; masked by the caller).
template <class C>
__device__ __forceinline__ void copy_tile(const uint16_t* src, unsigned dst, int r0, int N, const BLane<C>& bl,
                                          int w) {
  if (r0 + C::T <= N) {
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
      const int t = w + C::NW * ii;
      const char* base = (const char*)src + ((size_t)r0 + (size_t)t * C::RPI) * C::ROWB;
      lds_copy16_s(base, bl.g, dst + t * 1024);
    }
  } else {
    int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
      const int t = w + C::NW * ii;
      const int row = t * C::RPI + lane / C::CPR;
      const int chunk = (lane % C::CPR) ^ swz<C::D>(row);
      const int grow = min(r0 + row, N - 1);
      lds_copy16(src + (size_t)grow * C::D + (size_t)chunk * 8, dst + t * 1024);
    }
  }
}

__device__ __forceinline__ bf16x8 lds_row(unsigned addr) {
  return *(const bf16x8 LDS_AS*)((const unsigned char LDS_AS*)0 + addr);
}

// Transposed operand of 16-row block kq, dim block db, of the tile at addr.
template <class C>
__device__ __forceinline__ bf16x8 lds_tr(const BLane<C>& bl, unsigned addr, int kq, int db) {
  const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
  const int off = kq * 16 * C::ROWB;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + addr + bl.tr[db][0] + off));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + addr + bl.tr[db][1] + off));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One work unit -> up to two tiles of rows (the causal pairing of a heavy
// and a light tile); the 1-D grid is remapped so that XCD x runs the
// contiguous units [x * per_xcd, (x + 1) * per_xcd).
__device__ __forceinline__ int unit_of_block(int per_xcd) {
  return (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
}

// Store the 32 x 32*DB block held in acc (lane: row l%32, regs: columns
// 8*(r/4) + 4*(l/32) + r%4 of each 32-column block) as bf16 rows, times mul.
template <class C>
__device__ __forceinline__ void store_rows(uint16_t* rowp, const f32x16 (&acc)[C::DB], float mul, int h) {
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[db][4 * a + e] * mul);
      *(u32x2*)(rowp + 32 * db + 8 * a + 4 * h) = __builtin_bit_cast(u32x2, ov);
    }
}

// ---------------------------------------------------------------------------
// dQ kernel: query-tiled.  Also writes D_i = O_i . dO_i for its rows.
template <class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                 const uint16_t* __restrict__ o, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
                 uint16_t* __restrict__ dq, float* __restrict__ delta, int N, int T_r, int units_per_head,
                 int num_units, int per_xcd, int pair, float c, float scale, unsigned ssign) {
  // a ring of DQ_NST stages of (K, V) tiles: copies run two tiles ahead
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DQ_NST * C::DQSTAGE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int u = unit_of_block(per_xcd);
  if (u >= num_units) return;
  const int bh = u / units_per_head;
  const int ur = u - bh * units_per_head;
  // causal pairs: the heavy query tile T_r-1-ur, then the light tile ur
  int tiles[2] = {(CAUSAL && pair) ? T_r - 1 - ur : ur, ur};
  const int ntiles = (CAUSAL && pair && tiles[1] < tiles[0]) ? 2 : 1;

  BLane<C> bl;
  blane<C>(bl, w, lane);
  const unsigned lbase = (unsigned)(uintptr_t)(const unsigned char LDS_AS*)smem;
  const size_t hoff = (size_t)bh * (size_t)N * C::D;
  int rowa[C::KB], tra[C::DB][2];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) rowa[kb] = (int)lbase + bl.row[kb];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    tra[db][0] = (int)lbase + bl.tr[db][0];
    tra[db][1] = (int)lbase + bl.tr[db][1];
  }

  for (int ti = 0; ti < ntiles; ++ti) {
    const int q0 = tiles[ti] * C::ROWS;
    const int query = q0 + w * 32 + l32;
    const int qrow = min(query, N - 1);

    // Q and dO rows as register operands (lane: query l%32, dims
    // 16 kb + 8 (l/32) .. +7); D_i = O_i . dO_i in fp32
    bf16x8 qr[C::KB], dor[C::KB];
    float dsum = 0.f;
    {
      const size_t ro = hoff + (size_t)qrow * C::D + 8 * h;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        qr[kb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(q + ro + 16 * kb) ^ ssign);
        dor[kb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(dout + ro + 16 * kb));
        const bf16x8 ov = __builtin_bit_cast(bf16x8, *(const u32x4*)(o + ro + 16 * kb));
#pragma unroll
        for (int j = 0; j < 8; ++j) dsum = fmaf((float)ov[j], (float)dor[kb][j], dsum);
      }
    }
    const float dval = half_sum(dsum);
    if (h == 0 && query < N) delta[(size_t)bh * N + query] = dval;
    const float l2 = lse[(size_t)bh * N + qrow] * kLog2e;

    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + C::ROWS) : N;
    const int nkv = (kv_end + C::T - 1) / C::T;
    // tiles before nfull need no mask for any query of the workgroup
    int nfull = N / C::T;
    if (CAUSAL) nfull = min(nfull, (q0 + 1) / C::T);

    const uint16_t* kh = k + hoff;
    const uint16_t* vh = v + hoff;
    auto issue = [&](int j) __attribute__((always_inline)) {
      const unsigned st = lbase + (unsigned)(j % DQ_NST) * C::DQSTAGE;
      copy_tile<C>(kh, st, j * C::T, N, bl, w);
      copy_tile<C>(vh, st + C::TB, j * C::T, N, bl, w);
    };
    // dP^T starts from -D, so that the accumulator ends as dP^T - D
    f32x16 negd;
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = -dval;
    const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
    // dQ^T += K^T dS^T for the tile in stage ST (K^T by transpose reads)
    auto dq_mfma = [&](auto stc, const bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
      constexpr int KT = decltype(stc)::value * C::DQSTAGE;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int off = KT + kq * 16 * C::ROWB;
          const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][0] + off));
          const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][1] + off));
          const bf16x8 kt = __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = mfma(kt, dsb[kq], acc[db]);
        }
    };
    // Step j (stage ST = j % 4, compile-time, so that every LDS address is a
    // per-lane offset with the LDS base folded in, plus an immediate): the
    // products of tile j (S^T, dP^T) together with the dQ product of tile
    // j - 1, whose dS^T the previous step left in dsp; then the softmax
    // gradient of tile j into dsp.  Copies run two tiles ahead; a stage is
    // refilled only after the step that last read it (dQ of its tile).
    bf16x8 dsp[2];
    auto step = [&](int j, auto stc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value;
      constexpr int KT = ST * C::DQSTAGE, VT = KT + C::TB;
      if (j + 2 < nkv) issue(j + 2);
      // S^T = K Q^T and dP^T - D = V dO^T - D (lane: query l%32; regs: keys
      // 8*(r/4) + 4h + r%4)
      f32x16 s = {}, dp = negd;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        s = mfma(*(const bf16x8 LDS_AS*)(lds + rowa[kb] + KT), qr[kb], s);
        dp = mfma(*(const bf16x8 LDS_AS*)(lds + rowa[kb] + VT), dor[kb], dp);
      }
      if (j > 0) dq_mfma(std::integral_constant<int, (ST + DQ_NST - 1) % DQ_NST>{}, dsp);
      // a masked score becomes -inf: weight exp2(-inf) = 0 exactly (c > 0)
      if (j >= nfull) {  // wave-uniform: the diagonal and ragged tiles only
        const int lim = (CAUSAL ? min(query, N - 1) : N - 1) - (j * C::T + 4 * h);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) > lim) s[i] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dsp[i >> 3][i & 7] = (__bf16)(__builtin_amdgcn_exp2f(fmaf(s[i], c, -l2)) * dp[i]);
      // tile j + 1 has landed (tile j + 2 may still be in flight); the
      // barrier also orders every read of this step before later refills
      if (j + 2 < nkv) wait_copies<2 * C::NI>();
      else wait_copies<0>();
      barrier();
    };
    issue(0);
    if (1 < nkv) {
      issue(1);
      wait_copies<2 * C::NI>();
    } else {
      wait_copies<0>();
    }
    barrier();
    int j = 0;
    for (; j + 3 < nkv; j += 4) {
      step(j, std::integral_constant<int, 0>{});
      step(j + 1, std::integral_constant<int, 1>{});
      step(j + 2, std::integral_constant<int, 2>{});
      step(j + 3, std::integral_constant<int, 3>{});
    }
    // the remaining tiles, then the dQ product of the last one
    const int rem = nkv - j;
    if (rem > 0) step(j, std::integral_constant<int, 0>{});
    if (rem > 1) step(j + 1, std::integral_constant<int, 1>{});
    if (rem > 2) step(j + 2, std::integral_constant<int, 2>{});
    if (rem == 0) dq_mfma(std::integral_constant<int, 3>{}, dsp);
    else if (rem == 1) dq_mfma(std::integral_constant<int, 0>{}, dsp);
    else if (rem == 2) dq_mfma(std::integral_constant<int, 1>{}, dsp);
    else dq_mfma(std::integral_constant<int, 2>{}, dsp);
    barrier();  // every wave is done with the ring before the next tile refills it
    if (query < N) store_rows<C>(dq + hoff + (size_t)query * C::D, acc, scale, h);
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel: key-tiled.
template <class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const float* __restrict__ lse,
                   const uint16_t* __restrict__ dout, const float* __restrict__ delta, uint16_t* __restrict__ dk,
                   uint16_t* __restrict__ dv, int N, int T_r, int units_per_head, int num_units, int per_xcd,
                   int pair, float c, float scale, unsigned ssign) {
  // two stages of (Q, dO, L, D) tiles, then the V rows of the workgroup's keys
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * C::STAGE + C::ROWS * C::ROWB];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int u = unit_of_block(per_xcd);
  if (u >= num_units) return;
  const int bh = u / units_per_head;
  const int ur = u - bh * units_per_head;
  // causal pairs: key tile ur (it sees more queries), then T_r-1-ur
  int tiles[2] = {ur, (CAUSAL && pair) ? T_r - 1 - ur : ur};
  const int ntiles = (CAUSAL && pair && tiles[1] > tiles[0]) ? 2 : 1;

  BLane<C> bl;
  blane<C>(bl, w, lane);
  const unsigned lbase = (unsigned)(uintptr_t)(const unsigned char LDS_AS*)smem;
  const size_t hoff = (size_t)bh * (size_t)N * C::D;
  // per-lane LDS addresses with the base folded in (streamed tiles: + stage
  // immediates; the resident V rows of this wave: + a wave-uniform offset)
  int rowa[C::KB], tra[C::DB][2];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) rowa[kb] = (int)lbase + bl.row[kb];
  const int vw = 2 * C::STAGE + w * C::TB;  // this wave's resident V rows, from the base
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    tra[db][0] = (int)lbase + bl.tr[db][0];
    tra[db][1] = (int)lbase + bl.tr[db][1];
  }
  const int xa = (int)lbase;
  const float* lh = lse + (size_t)bh * N;
  const float* dh = delta + (size_t)bh * N;

  for (int ti = 0; ti < ntiles; ++ti) {
    const int k0 = tiles[ti] * C::ROWS;
    const int key = k0 + w * 32 + l32;
    const int krow = min(key, N - 1);

    // K rows as register operands (lane: key l%32, dims 16 kb + 8h ..); the
    // V rows of the workgroup's keys go to LDS (32-row tile w holds wave w's)
    bf16x8 kr[C::KB];
    {
      const size_t ro = hoff + (size_t)krow * C::D + 8 * h;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        kr[kb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(k + ro + 16 * kb) ^ ssign);
    }
    const unsigned vres = lbase + 2 * C::STAGE;
#pragma unroll
    for (int t = 0; t < C::NW; ++t) copy_tile<C>(v + hoff, vres + t * C::TB, k0 + t * C::T, N, bl, w);
    f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dka[db][i] = 0.f;
        dva[db][i] = 0.f;
      }

    // query tiles that can see a key of this workgroup
    const int qt0 = CAUSAL ? k0 / C::T : 0;
    const int nq = (N + C::T - 1) / C::T;
    // query tiles from qfull on need no mask for any key of the workgroup
    const int qfull = CAUSAL ? (k0 + C::ROWS + C::T - 1) / C::T : 0;

    const uint16_t* qh = q + hoff;
    const uint16_t* oh = dout + hoff;
    // stage of query tile i: (i - qt0) & 1
    // Wave 0 loads L (lanes 0..31) and D (lanes 32..63) of the tile's 32
    // queries into a register when the tile's copies are issued, and writes
    // them to LDS (L times log2(e), once per query instead of once per lane
    // that uses it) after its copies have landed, before the barrier that
    // publishes the tile.
    float lx = 0.f;
    auto issue = [&](int i) __attribute__((always_inline)) {
      const unsigned st = lbase + (unsigned)((i - qt0) & 1) * C::STAGE;
      copy_tile<C>(qh, st, i * C::T, N, bl, w);
      copy_tile<C>(oh, st + C::TB, i * C::T, N, bl, w);
      if (w == 0) {
        const int r = min(i * C::T + l32, N - 1);
        lx = h ? dh[r] : lh[r];
      }
    };
    auto publish = [&](int i) __attribute__((always_inline)) {
      if (w == 0) {
        const unsigned st = lbase + (unsigned)((i - qt0) & 1) * C::STAGE;
        *(float LDS_AS*)((unsigned char LDS_AS*)0 + st + 2 * C::TB + 4 * lane) = h ? lx : lx * kLog2e;
      }
    };
    issue(qt0);
    wait_copies<0>();
    publish(qt0);
    barrier();
    // V rows negated in place (once per key tile), so that dP - D comes out
    // of the matrix cores as D + dO (-V)^T with the accumulator started at D
    {
      unsigned char LDS_AS* vb = (unsigned char LDS_AS*)0 + vres;
#pragma unroll
      for (int e = 0; e < C::NW * C::TB / (16 * C::NW * 64); ++e) {
        u32x4 LDS_AS* p = (u32x4 LDS_AS*)(vb + 16 * (threadIdx.x + C::NW * 64 * e));
        *p = *p ^ 0x80008000u;
      }
    }
    barrier();
    const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
    // masked: tiles holding the diagonal (before qfull) and a ragged last tile
    auto masked = [&](int i) __attribute__((always_inline)) { return i < qfull || i * C::T + C::T > N; };
    // One query tile; stage ST and the mask are compile-time, so every LDS
    // address is a per-lane offset (LDS base folded in) plus an immediate.
    auto step = [&](int i, auto stc, auto maskc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value;
      constexpr bool MASK = decltype(maskc)::value;
      constexpr int QT = ST * C::STAGE, OT = QT + C::TB, XT = QT + 2 * C::TB;
      if (i + 1 < nq) issue(i + 1);
      // D of this lane's 16 queries starts the dP accumulator
      f32x16 dp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b = *(const f32x4 LDS_AS*)(lds + xa + XT + 128 + (8 * g + 4 * h) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * g + e] = b[e];
      }
      // S = Q K^T and D - dP = D + dO (-V)^T (lane: key l%32; regs:
      // queries 8*(r/4) + 4h + r%4 of the tile)
      f32x16 s = {};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        s = mfma(*(const bf16x8 LDS_AS*)(lds + rowa[kb] + QT), kr[kb], s);
        dp = mfma(*(const bf16x8 LDS_AS*)(lds + rowa[kb] + OT), *(const bf16x8 LDS_AS*)(lds + rowa[kb] + vw), dp);
      }
      // register r holds query q0 + 4h + rel, rel = 8*(r/4) + r%4: visible
      // iff rel <= N - 1 - (q0 + 4h) and (causal) rel >= key - (q0 + 4h)
      // a masked score becomes -inf: weight exp2(-inf) = 0 exactly (c > 0)
      if (masked(i)) {  // wave-uniform: only diagonal and ragged tiles
        // register r holds query q0 + 4h + rel, rel = 8*(r/4) + r%4: visible
        // iff rel <= N - 1 - (q0 + 4h) and (causal) rel >= key - (q0 + 4h)
        const int qb = i * C::T + 4 * h;
        const int rhi = N - 1 - qb, rlo = CAUSAL ? key - qb : -1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 8 * (r >> 2) + (r & 3);
          if (rel > rhi || rel < rlo) s[r] = -INFINITY;
        }
      }
      // P from L (log2 units) of the lane's 16 queries (read from LDS four
      // at a time, next to their use)
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lg = *(const f32x4 LDS_AS*)(lds + xa + XT + (8 * g + 4 * h) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lg[e]));  // (L in log2 units)
          pb[r >> 3][r & 7] = (__bf16)pv;
          dsb[r >> 3][r & 7] = (__bf16)(pv * dp[r]);  // -dS
        }
      }
      // dV^T += dO^T P and -dK^T += Q^T (-dS) (dO^T and Q^T by transpose reads)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int off = kq * 16 * C::ROWB;
          const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][0] + OT + off));
          const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][1] + OT + off));
          const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][0] + QT + off));
          const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + tra[db][1] + QT + off));
          const bf16x8 ot = __builtin_shufflevector(__builtin_bit_cast(bf16x4, a0), __builtin_bit_cast(bf16x4, a1),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 qt = __builtin_shufflevector(__builtin_bit_cast(bf16x4, b0), __builtin_bit_cast(bf16x4, b1),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          dva[db] = mfma(ot, pb[kq], dva[db]);
          dka[db] = mfma(qt, dsb[kq], dka[db]);
        }
      wait_copies<0>();
      if (i + 1 < nq) publish(i + 1);
      barrier();
    };
    int i = qt0;
    for (; i + 1 < nq; i += 2) {
      step(i, std::integral_constant<int, 0>{}, std::false_type{});
      step(i + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
    if (i < nq) step(i, std::integral_constant<int, 0>{}, std::false_type{});
    if (key < N) {
      store_rows<C>(dk + hoff + (size_t)key * C::D, dka, -scale, h);  // dka holds -dK^T / scale
      store_rows<C>(dv + hoff + (size_t)key * C::D, dva, 1.f, h);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              const void* dq, const void* dk, const void* dv, const float* delta, int B, int H, int N, int d,
              float scale) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const long long rows = (long long)B * H * N;
  if (rows == 0) return FA_OK;
  if ((long long)B * H > (1LL << 30) || rows > (1LL << 40)) return FA_ERR_SHAPE;
  if ((long long)B * H * ((N + 127) / 128) > (1LL << 30)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return FA_ERR_ALIGN;
  const size_t nb = (size_t)rows * d * 2;
  const size_t lb = (size_t)rows * sizeof(float);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t insz[6] = {nb, nb, nb, nb, nb, lb};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t outsz[4] = {nb, nb, nb, lb};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], outsz[a], ins[b], insz[b])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], outsz[a], outs[b], outsz[b])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

template <class C, bool CAUSAL>
void launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int N, float c, float scale,
                unsigned ssign, hipStream_t stream) {
  const int T = (N + C::ROWS - 1) / C::ROWS;
  // causal units pair a heavy tile with a light one when there are more
  // tiles than the 256 CUs; with fewer, every tile gets a CU of its own (two
  // unpaired heavy tiles sharing one CU were slower than their pairs)
  const int pair = CAUSAL && (long long)B * H * T > 256;
  const int units_per_head = pair ? (T + 1) / 2 : T;
  const int num_units = B * H * units_per_head;
  const int per_xcd = (num_units + 7) / 8;
  const int grid = per_xcd * 8;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<C, CAUSAL>), dim3(grid), dim3(C::NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o, lse,
                     (const uint16_t*)dout, (uint16_t*)dq, delta, N, T, units_per_head, num_units, per_xcd, pair,
                     c, scale, ssign);
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<C, CAUSAL>), dim3(grid), dim3(C::NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, lse, (const uint16_t*)dout,
                     (const float*)delta, (uint16_t*)dk, (uint16_t*)dv, N, T, units_per_head, num_units, per_xcd,
                     pair, c, scale, ssign);
}

}  // namespace

extern "C" int fa_bwd_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, const void* dq, const void* dk, const void* dv,
                                 const float* delta, int B, int H, int N, int d, float scale, int causal) {
  (void)causal;
  return check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d,
                      float scale, int causal, hipStream_t stream) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale);
  if (st != FA_OK) return st;
  if ((long long)B * H * N == 0) return FA_OK;
  // The scores are formed as |scale| * (sign(scale) Q) K^T: the dQ kernel
  // flips the sign bits of its register Q rows, the dK/dV kernel those of
  // its register K rows (exact), so that the kernels see c > 0 (a masked
  // score of -inf then has weight exactly 0).  dQ and dK keep the signed
  // scale.  A zero scale runs as 2^-100, as in the forward (every
  // exponent argument rounds to -L log2(e), i.e. P = exp(-L)).
  const unsigned ssign = (scale < 0.f) ? 0x80008000u : 0u;
  const float c = scale == 0.f ? 0x1p-100f : fabsf(scale) * kLog2e;
  if (d == 128) {
    if (causal)
      launch_bwd<BCfg<128>, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, c, scale, ssign, stream);
    else
      launch_bwd<BCfg<128>, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, c, scale, ssign, stream);
  } else {
    if (causal)
      launch_bwd<BCfg<64>, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, c, scale, ssign, stream);
    else
      launch_bwd<BCfg<64>, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, c, scale, ssign, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
