// Exact attention forward for MI355X (gfx950, CDNA4): HIP kernels + C ABI.
//
// What is computed (per batch b, head h; square self-attention):
//   O = softmax(scale * Q K^T [causal: key j visible to query i iff j <= i]) V
//   LSE = m + ln(l), the natural-log logsumexp of each query row's scores.
// Sources: "Lecture 3 - FlashAttention-1 Algorithm" (jared-hpc.com), section
// "The forward loop (Algorithm 1 from the FA1 paper)": Q-outer, KV-inner loop
// with running m and l, O and LSE written once per query tile.  "15.
// FlashAttention" (inference.shantanugoel.com), section "Online softmax:
// normalize as you go" (unnormalised accumulator a, O = a / l) and section
// "The kernel" (one program per query block of one (batch, head), the causal
// loop bound, the safe reference for a row with no visible key yet, masked
// tail loads, fp32 statistics with p cast to the value type for P V).
// "FlashAttention：从 IO-Aware Attention 到 GPU Work Partitioning"
// (blog.euler0525.cn), sections "Sequence Parallelism" (query tiles are the
// parallel work units), "Warp Work Partitioning" (each wave owns its own
// query rows; no cross-wave reduction of O) and "Tile Size 与 Causal
// Attention" (tiles above the diagonal are skipped, only diagonal tiles are
// masked element by element).
//
// gfx950 design (one workgroup = 8 wave64s, each wave owns 32 query rows):
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16.  In the MFMA accumulator layout a lane then
//    holds ONE query (lane % 32) and 16 keys per 32-key block, so the row
//    max / row sum are in-lane reductions plus one v_permlane32_swap, and the
//    per-row rescale factor is a per-lane scalar.
//  * The same accumulator registers, rounded to bf16, are directly the B
//    operand of O^T = V^T P^T (no data movement for P).  The V^T operand is
//    read from a row-major V tile in LDS with ds_read_b64_tr_b16, the gfx950
//    LDS transpose load.
//  * K and V tiles are copied HBM -> LDS with global_load_lds_dwordx4
//    (no VGPR staging) into a ring of four LDS stages, issued two (d = 64)
//    or three (d = 128) tiles ahead of their use, with an XOR swizzle of the
//    16-byte chunks so that both the K reads and the transposed V reads hit
//    distinct LDS banks.
//  * Each step of a wave is a matrix-core phase (S_j = K_j Q^T and
//    acc += V_{j-1}^T P_{j-1}^T) and a vector-ALU phase (softmax of S_j).
//    The two waves of a SIMD run one phase apart, so one feeds the matrix
//    cores while the other computes exponentials (d = 128: one workgroup
//    barrier per step; d = 64: one per phase).  In the matrix phase
//    every LDS address is a per-lane offset computed once plus an
//    immediate, so that phase issues no address arithmetic.  At d = 64,
//    where the softmax of 128 keys is the longer phase, the bf16 packing of
//    P_{j-1} (and its normaliser correction, below) moves into the matrix
//    phase, beside the first products of S_j.
//  * The exponent reference of a row is fixed after its first key tile, so
//    the loop normally rescales nothing; a wave whose weights outgrow it by
//    more than 2^16 in a tile takes the running-max step of the recurrence
//    for that tile (new reference, acc and l rescaled, weights formed
//    again), so the weights stay bounded.
//  * Exponentials are exp2 with log2(e) folded into the scale; m, l and the
//    output accumulator stay in fp32 registers; O is divided once, by the
//    sum of the bf16 weights that P V multiplied (l plus a correction taken
//    on the tiles that dominate a row), and staged through LDS, so that its
//    global stores are whole rows.
//  * Work units are query tiles (causal: a heavy tile paired with a light
//    one, so every unit costs the same); the 1-D grid is remapped so that
//    each XCD runs a contiguous range of units, i.e. the query tiles of the
//    same heads, which then share K/V through that XCD's L2.
//
// The fp32 entry point (fa_fwd_f32.hip) and the split-KV entry point with
// its small-tile and merge kernels (fa_split.hip) live in their own files;
// split-KV's large-tile form is the split mode of this file's kernel.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_host.h"

namespace {

using namespace fa;

// Exponent reference.  A row's reference m is the max of its first key
// tile with a visible key, and later unmasked tiles compute no max: their
// weights are p = exp2(s*c - m) against that fixed m.  O = acc / l and
// LSE = m + log2 l are the same for any common reference in exact
// arithmetic (the running max of the recurrence only bounds the exponents),
// so this equals the pages' recurrence as long as the weights stay bounded.
// They are kept <= 2^kSlack: when the weights one lane sums for a tile
// exceed 2^kSlack (a score rose more than kSlack above the reference, or an
// exponential overflowed), or a masked tile's max rises more than kSlack
// above it, the wave takes the recurrence's step for that tile -- the new
// reference is the running max, l and acc are multiplied by
// exp2(m_old - m_new), and the tile's weights are formed again.  Then
// l <= N * 2^kSlack and |acc| <= N * 2^kSlack * max|V|.
constexpr float kSlack = 16.0f;
constexpr float kJumpSum = 0x1p16f;  // 2^kSlack

// ---------------------------------------------------------------------------
// Tile configuration of the bf16 kernel: NW waves of 32 query rows each
// (8: two waves per SIMD), key tiles of BC rows, a ring of NST LDS stages.
// LDS layout: the K tiles of the NST stages, then the V tiles.
template <int D_, int BC_, int NW_ = 8>
struct Cfg {
  static constexpr int D = D_;             // head dimension
  static constexpr int BC = BC_;           // keys per K/V tile (B_c)
  static constexpr int NW = NW_;           // waves per workgroup
  static constexpr int BR = 32 * NW;       // query rows per tile (B_r)
  static constexpr int ROWB = D * 2;       // bytes of one K/V row
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;     // rows per 1 KB wave-wide copy
  static constexpr int KT = BC * ROWB;     // bytes of one K (or V) tile
  static constexpr int NST = 4;            // LDS stages of the K/V ring
  static constexpr int VBASE = NST * KT;   // start of the V tiles in LDS
  static constexpr int LDSB = 2 * NST * KT;
  static constexpr int NINST = KT / 1024;  // 1 KB copies per matrix per tile
  static constexpr int NCW = NW / 2;       // waves copying one matrix (K: the first half, V: the second)
  static_assert(NW == 4 || NW == 8, "workgroup of 4 or 8 waves");
  static constexpr int NI = NINST / NCW;   // copy instructions per wave per tile
  static constexpr int KB = D / 16;        // 16-deep k-steps of Q K^T
  static constexpr int DB = D / 32;        // 32-dim output blocks
  static constexpr int SB = BC / 32;       // 32-key score blocks
  static constexpr int PB = BC / 16;       // 16-key k-steps of P V
  static_assert(NINST % NCW == 0 && NI >= 1, "copy instructions must split evenly over waves");
  static_assert(NI <= 15, "copies of one tile must fit the wait counter");
  static constexpr int KD = 2;             // K operands read ahead, in k-steps
  // Where the global -> LDS copies go: true = in the vector phase, three
  // tiles ahead (d = 128, where the matrix phase is the longer one); false =
  // at the start of the matrix phase, two tiles ahead (d = 64, where the
  // softmax of BC = 128 keys is the longer one).
  static constexpr bool VCOPY = D == 128;
  static_assert((NCW * RPI) % 16 == 0, "a wave's copy rows must be a swizzle period apart");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  // stage offsets are folded into the 16-bit offset field of the LDS reads
  static_assert((NST - 1) * KT + (SB - 1) * 32 * ROWB < 65536, "K read offset range");
  static_assert((NST - 1) * KT + (PB - 1) * 16 * ROWB < 65536, "V read offset range");
  // The epilogue stages each wave's O tile (32 rows x D, bf16) in LDS so that
  // its global stores are whole rows.  The staging area starts at V stage 2:
  // the next query tile's first copies fill only K stages 0..2 and V stages
  // 0..1 before its first barrier, so the area is free until every wave has
  // passed that barrier, i.e. finished its epilogue.
  static constexpr int OBASE = VBASE + 2 * KT;
  static constexpr int OROWS = 32 * ROWB;                  // one wave's staged O tile
  static constexpr int LDS_TOTAL = OBASE + BR * ROWB > LDSB ? OBASE + BR * ROWB : LDSB;
  static_assert(NST == 4 && (VCOPY ? 3 : 2) <= 3, "prologue copies stay below the staging area");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS size");
};


// Per-lane LDS and copy offsets, computed once per workgroup.
// Waves 0..NCW-1 copy the K tiles, waves NCW..2NCW-1 the V tiles.  Copy
// instruction ii of wave w moves the 1 KB block t = w % NCW + NCW * ii of
// its matrix, i.e. tile rows RPI*t .. RPI*t + RPI-1 (to LDS bytes 1024 t ..);
// consecutive instructions of a wave are NCW*RPI rows apart, a multiple of
// the swizzle period, so one lane offset serves them all and the rest is a
// wave-uniform base.
template <class C>
struct LaneOffsets {
  int k[C::KB];        // K operand of k-step kb: row l%32, dims 16kb + 8(l/32) .. +7
  int v[C::DB][2];     // V^T operand of output block db, rows +0 / +8 (see tile_m)
  unsigned g;          // copies: byte offset of this lane's 16 bytes within block w
  unsigned base;       // LDS address of the K/V ring
};

template <class C>
__device__ __forceinline__ void lane_offsets(LaneOffsets<C>& lo, unsigned base, int w, int lane) {
  lo.base = base;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kf = swz<C::D>(l32);
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) lo.k[kb] = (int)base + l32 * C::ROWB + 16 * ((2 * kb + h) ^ kf);
  // V^T via LDS transpose loads: lane (g = l/16, r, b) reads V row (16*kb2 +
  // 4h + r [+8]), dims (32*db + 16*(g%2) + 4b .. +3); after the transpose,
  // lane l holds V[16*kb2 + 4h + 0..3 (+8)][32*db + l%32].
  const int vr = 4 * h + ((lane >> 2) & 3);
  const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vf0 = swz<C::D>(vr), vf1 = swz<C::D>(vr + 8);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int dim = 32 * db + vdim;
    lo.v[db][0] = (int)base + C::VBASE + vr * C::ROWB + 16 * ((dim >> 3) ^ vf0) + 2 * (dim & 7);
    lo.v[db][1] = (int)base + C::VBASE + (vr + 8) * C::ROWB + 16 * ((dim >> 3) ^ vf1) + 2 * (dim & 7);
  }
  const int row = (w % C::NCW) * C::RPI + lane / C::CPR;  // row of block w % NCW
  const int chunk = (lane % C::CPR) ^ swz<C::D>(row);
  lo.g = (unsigned)(lane / C::CPR * C::ROWB + chunk * 16);
}

// This wave's HBM -> LDS copies of its matrix (K for waves 0..NCW-1, V for
// the others; src is that matrix of the head) for tile k0 .. k0+BC-1, into
// the stage at byte offset st.  A full tile uses a scalar base and the
// fixed lane offset; the last tile of a sequence whose length is not a
// multiple of BC clamps rows past the end to row N-1 (never read past the
// array, finite, masked to -inf in K and multiplied by an exact 0 in V).
template <class C>
__device__ __forceinline__ void load_tile(const uint16_t* src, unsigned lds_st, int k0, int N,
                                          const LaneOffsets<C>& lo, int w) {
  const int wc = w % C::NCW;
  if (k0 + C::BC <= N) {
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
      const int t = wc + C::NCW * ii;
      const char* base = (const char*)src + ((size_t)k0 + (size_t)t * C::RPI) * C::ROWB;
      lds_copy16_s(base, lo.g, lds_st + t * 1024);
    }
  } else {
    // (the lane index is made opaque so that the compiler recomputes these
    // rarely used addresses here instead of keeping them live in registers)
    int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
      const int t = wc + C::NCW * ii;
      const int row = t * C::RPI + lane / C::CPR;
      const int chunk = (lane % C::CPR) ^ swz<C::D>(row);
      const int grow = min(k0 + row, N - 1);
      lds_copy16(src + (size_t)grow * C::D + (size_t)chunk * 8, lds_st + t * 1024);
    }
  }
}

// K operand of k-step kb, 32-key block sb, of the K tile at stage offset kst.
template <class C>
__device__ __forceinline__ bf16x8 lds_k(const LaneOffsets<C>& lo, int kst, int kb, int sb) {
  const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
  return *(const bf16x8 LDS_AS*)(lds + lo.k[kb] + (kst + sb * 32 * C::ROWB));
}

// The K operands of the first KD k-steps of the tile at stage offset kst,
// read ahead of the matrix phase that uses them.
template <class C>
__device__ __forceinline__ void prefetch_k(bf16x8 (&kpre)[C::KD][C::SB], const LaneOffsets<C>& lo, int kst) {
#pragma unroll
  for (int kb = 0; kb < C::KD; ++kb)
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) kpre[kb][sb] = lds_k<C>(lo, kst, kb, sb);
}

// A lane's running sums over its keys of a row: lh = l / 2, where l is the
// sum of the unrounded fp32 weights (LSE = m + log2 l; kept halved, an exact
// scaling, so that the heavy-tile test below is one compare), and
// corr = sum of (bf16(p) - p) over the tiles where it was taken.  O divides
// by l + corr, the sum of the bf16 weights that P V multiplies, so that a
// row dominated by one key gets that key's V row up to the bf16 rounding
// of O.  (With the reference fixed at the first tile's max, a dominant
// later weight is 2^rise, not 1 as under the running max: dividing by the
// unrounded l would carry its bf16 rounding, up to 2^-8 relative, into O.)
// The correction is taken on a tile only when the lane's weights of the
// tile exceed half of what it summed before (a "heavy" tile; the branch is
// wave-uniform, the correction per lane): a weight of a tile left out is
// less than half of its row's final sum, so its rounding moves O by less
// than 2^-9 |v|, and the weights that dominate a row are always corrected.
struct RowSums {
  float lh, corr;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// P (fp32, in the score registers of block sb) to the bf16 operand of P V.
template <class C>
__device__ __forceinline__ void pack_block(const f32x16 (&s)[C::SB], bf16x8 (&pb)[C::PB], int sb) {
#pragma unroll
  for (int kb2 = 2 * sb; kb2 < 2 * sb + 2; ++kb2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[kb2][j] = (__bf16)s[kb2 >> 1][8 * (kb2 & 1) + j];
    pin(pb[kb2]);
  }
}

// A tile's bf16 rounding correction of the normaliser (see RowSums): on a
// heavy tile, corr += (sum of the bf16 weights) - ts, where ts is the sum of
// the unrounded weights.  The branch is wave-uniform, the correction per
// lane (a row's bits never depend on other rows).
template <class C>
__device__ __forceinline__ void heavy_corr(const bf16x8 (&pb)[C::PB], float ts, bool heavy, RowSums& sums) {
  if (__builtin_amdgcn_ballot_w64(heavy) != 0) {
    // sum of the bf16 weights, v_dot2c_f32_bf16 against (1, 1)
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float tb[2] = {0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < C::PB; ++kb2) {
      tb[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kb2], pb[kb2], 0, 1), one2, tb[0], false);
      tb[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kb2], pb[kb2], 2, 3), one2, tb[1], false);
      tb[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kb2], pb[kb2], 4, 5), one2, tb[0], false);
      tb[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kb2], pb[kb2], 6, 7), one2, tb[1], false);
    }
    sums.corr += heavy ? (tb[0] + tb[1]) - ts : 0.f;
  }
}

// A tile's weights not yet packed: the matrix phase that multiplies them
// packs them and takes the heavy-tile correction (the two-barrier schedule,
// d = 64, where the softmax is the longer phase).
struct PendingP {
  float ts;    // this lane's sum of the tile's unrounded weights
  bool heavy;  // ts > half of what the lane summed before the tile
};

// The matrix-core phase of one step: S = K Q^T (HAS_QK, K tile at stage
// offset kst) and acc += V^T P^T (HAS_PV, V tile at stage offset vst).
// LDS operands are read a few MFMAs ahead of their use (two k-steps for K,
// four operands for V), and scheduling barriers keep that order, so that
// the LDS latency hides behind the matrix cores; the first KD k-steps of K
// come in kpre, read during the preceding phase.  With kst / vst known at
// compile time, every LDS address is a precomputed lane offset plus an
// immediate: this phase issues no address arithmetic and no copy.
// PACKIN (with HAS_PV): s arrives holding the fp32 weights of the previous
// tile, which this phase packs into pb (each score block just before the
// first product that overwrites it) and corrects the normaliser for
// (heavy_corr), so that the vector phase, the longer one at d = 64, ends
// with the exponentials and their sum.
template <class C, bool HAS_QK, bool HAS_PV, bool PACKIN = false>
__device__ __forceinline__ void tile_m(int kst, int vst, const LaneOffsets<C>& lo, const bf16x8 (&qr)[C::KB],
                                       f32x16 (&s)[C::SB], bf16x8 (&pb)[C::PB], f32x16 (&acc)[C::DB],
                                       const bf16x8 (&kpre)[C::KD][C::SB], RowSums& sums, const PendingP& pend) {
  const unsigned char LDS_AS* lds = (const unsigned char LDS_AS*)0;
  auto load_k = [&](int kb, int sb) -> bf16x8 { return lds_k<C>(lo, kst, kb, sb); };
  constexpr int NV = C::PB * C::DB;  // V operands (one per P V instruction)
  auto load_v = [&](int i) -> bf16x8 {
    const int kb2 = i / C::DB, db = i % C::DB;
    const int off = vst + kb2 * 16 * C::ROWB;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + lo.v[db][0] + off));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(lds + lo.v[db][1] + off));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4, 5,
                                   6, 7);
  };
  constexpr int KD = C::KD;  // K prefetch distance in k-steps
  constexpr int VD = 4;      // V prefetch distance in operands
  bf16x8 ka[C::KB][C::SB];
  bf16x8 va[NV];
  const f32x16 zero = {};
  if (HAS_QK) {
#pragma unroll
    for (int kb = 0; kb < KD && kb < C::KB; ++kb)
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) ka[kb][sb] = kpre[kb][sb];
  } else if (HAS_PV) {
#pragma unroll
    for (int i = 0; i < VD && i < NV; ++i) va[i] = load_v(i);
  }
  __builtin_amdgcn_sched_barrier(0);
  // PACKIN: s holds the previous tile's fp32 weights; each block is packed
  // into pb just before the first product of this tile overwrites it
  constexpr bool PK = PACKIN && HAS_PV;
  if (PK && !HAS_QK) {
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) pack_block<C>(s, pb, sb);
  }
  if (HAS_QK) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) {
        if (PK && kb == 0) pack_block<C>(s, pb, sb);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][sb], qr[kb], kb == 0 ? zero : s[sb], 0, 0, 0);
      }
      if (kb + KD < C::KB) {
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) ka[kb + KD][sb] = load_k(kb + KD, sb);
      } else if (HAS_PV) {
        // the last k-steps start the V reads
        const int i0 = (kb + KD - C::KB) * VD / KD, i1 = (kb + KD - C::KB + 1) * VD / KD;
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (i >= i0 && i < i1) va[i] = load_v(i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (PK) {
    heavy_corr<C>(pb, pend.ts, pend.heavy, sums);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (HAS_PV) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      acc[i % C::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[i / C::DB], acc[i % C::DB], 0, 0, 0);
      if (i + VD < NV) va[i + VD] = load_v(i + VD);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Row max of the score tile in fp32, both halves of the wave (four
// independent max chains over this half's keys, then one lane swap).
template <class C>
__device__ __forceinline__ float tile_rowmax(const f32x16 (&s)[C::SB]) {
  float mq[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) mq[r] = s[0][r];
#pragma unroll
  for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
    for (int i = (sb == 0 ? 4 : 0); i < 16; ++i) mq[i & 3] = __builtin_fmaxf(mq[i & 3], s[sb][i]);
  return half_max(__builtin_fmaxf(__builtin_fmaxf(mq[0], mq[1]), __builtin_fmaxf(mq[2], mq[3])));
}

// The recurrence's step ("15. FlashAttention", section "Online softmax:
// normalize as you go") for the rows with `up` set: the reference moves up
// to the running max m_new = max(m, mxs), and l and acc are multiplied by
// exp2(m - m_new).  Other rows keep every bit as it is, so that a row's
// result never depends on what other rows of its wave see.
template <class C>
__device__ __forceinline__ void raise_ref(bool up, float mxs, float& m, RowSums& sums, f32x16 (&acc)[C::DB]) {
  const float m_new = up ? __builtin_fmaxf(m, mxs) : m;
  const float alpha = m_new > m ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
  sums.lh *= alpha;
  sums.corr *= alpha;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
  m = m_new;
}

// P = exp2(S*c - mref) in place (masked scores give exp2(-inf) = 0); returns
// this lane's sum of the unrounded weights.
template <class C>
__device__ __forceinline__ float tile_exp(f32x16 (&s)[C::SB], float c, float mref) {
  float sq[4];
#pragma unroll
  for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[sb][i] = __builtin_amdgcn_exp2f(fmaf(s[sb][i], c, -mref));
      if (sb == 0 && i < 4) sq[i] = s[sb][i];
      else sq[i & 3] += s[sb][i];
    }
  return (sq[0] + sq[1]) + (sq[2] + sq[3]);
}

// The vector-ALU phase: online softmax of one tile.  Mask (MASK: keys past
// N, and keys after the query when causal, get -inf, i.e. weight exactly 0;
// with a sliding window (wnd > 0) also keys before query - wnd + 1),
// exponent reference, P = exp2(S*c - m_ref), row sum of the unrounded
// weights; PACK: P into the bf16 operand pb and, on heavy tiles, the bf16
// rounding correction into sums (otherwise both are left to the next matrix
// phase, with the tile's sum and heavy flag in pend).
//  * FIRST / MASK tiles compute their row max.  The reference is the max of
//    the row's first tile with a visible key (a row that has seen none yet
//    uses the safe reference 0); a row whose max in a masked tile rises more
//    than kSlack above it raises it (raise_ref, behind a wave-uniform
//    branch).
//  * Other tiles compute no max.  When the weights of either half of a row
//    sum to more than 2^kSlack (every weight above 2^kSlack, or an overflow
//    to +inf, implies that), the wave forms the tile's scores again
//    (rescore: S = K Q^T from the K tile still in LDS, the same bits), those
//    rows raise their reference to the running max, and every row forms its
//    weights again (unchanged bits for the other rows: same scores, same
//    reference).
template <class C, bool CAUSAL, bool MASK, bool FIRST, bool PACK, class Rescore>
__device__ __forceinline__ void tile_softmax(f32x16 (&s)[C::SB], bf16x8 (&pb)[C::PB], f32x16 (&acc)[C::DB],
                                             float& m, RowSums& sums, PendingP& pend, int k0, int qw0, int N,
                                             float c, int lane, int wnd, Rescore&& rescore) {
  const int l32 = lane & 31;
  const int h = lane >> 5;
  // register i of block sb holds key k0 + 32*sb + 8*(i/4) + 4h + i%4
  if (MASK) {
    const int query = qw0 + l32;  // the query's position
    const int lim = (CAUSAL ? min(query, N - 1) : N - 1) - (k0 + 4 * h);
    if (wnd > 0) {
      // sliding window: keys query - wnd + 1 .. query
      const int low = query - wnd + 1 - (k0 + 4 * h);
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rel = 32 * sb + 8 * (i >> 2) + (i & 3);
          s[sb][i] = (rel <= lim && rel >= low) ? s[sb][i] : -INFINITY;
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[sb][i] = (32 * sb + 8 * (i >> 2) + (i & 3) <= lim) ? s[sb][i] : -INFINITY;
    }
  }
  if (FIRST || MASK) {
    const float mx = tile_rowmax<C>(s);
    const float mxs = (mx == -INFINITY) ? -INFINITY : mx * c;  // c > 0
    const bool had_ref = m != -INFINITY;
    const bool up = had_ref && mxs > m + kSlack;  // (the same in both halves of a row)
    if (!FIRST && __builtin_amdgcn_ballot_w64(up) != 0) raise_ref<C>(up, mxs, m, sums, acc);
    // the reference is the max of the first tile with a visible key
    m = had_ref ? m : mxs;
  }
  // safe reference (a row with no visible key yet: 0); after its first
  // tile with a visible key, m is finite
  const float mref = (FIRST || MASK) ? ((m == -INFINITY) ? 0.f : m) : m;
  float ts = tile_exp<C>(s, c, mref);
  if (!FIRST && !MASK) {
    // (NaN-safe: a NaN sum, from NaN inputs, does not take the branch)
    if (__builtin_amdgcn_ballot_w64(ts > kJumpSum) != 0) {
      const bool up = half_max(ts) > kJumpSum;  // either half of the row
      rescore();
      const float mx = tile_rowmax<C>(s);
      raise_ref<C>(up, mx * c, m, sums, acc);
      ts = tile_exp<C>(s, c, m);
    }
  }
  const bool heavy = ts > sums.lh;
  if (PACK) {
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) pack_block<C>(s, pb, sb);
    heavy_corr<C>(pb, ts, heavy, sums);
  } else {
    // (packed, and corrected when heavy, by the next matrix phase)
    pend.ts = ts;
    pend.heavy = heavy;
  }
  sums.lh = fmaf(ts, 0.5f, sums.lh);  // (exact scaling by a power of two)
  pin(sums.lh);
  pin(sums.corr);
}

// Arguments of the variants (EXT = true): query rows T and key rows S per
// head, Hq query heads of which each group of `group` reads one K/V head,
// the position of query row 0 (causal), a sliding window (0: none) and
// whether work units pair a heavy and a light query tile (both launchers
// set it; the plain kernel reads only this field).  Split-KV
// (nsplit > 1): a work unit is (query tile, split); split g covers keys
// [g * chunk, (g + 1) * chunk) and writes its normalised fp32 partial O_g
// and LSE_g (-inf for a row with no visible key in the chunk) to
// ws_o [nsplit, BH, T, d] and ws_lse [nsplit, BH, T] (BH = B * Hq).
struct ExtArgs {
  int T, S, Hq, group, offset, window, pair;
  int nsplit, chunk, BH;
  float* ws_o;
  float* ws_lse;
};

// One work unit: its query tiles, each over its key tiles.  smem: the K/V
// ring.
template <class C, bool CAUSAL, bool EXT>
__device__ __attribute__((always_inline)) inline void
fwd_unit(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
         uint16_t* __restrict__ o, float* __restrict__ lse, int N, int T_r, int units_per_head, int num_units,
         int per_xcd, float c, unsigned int qsign, const ExtArgs& ex, unsigned char LDS_AS* smem) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // Workgroups are dispatched round-robin over the 8 XCDs: block b runs on
  // XCD b % 8.  Give XCD x the contiguous units [x*per_xcd, (x+1)*per_xcd).
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= num_units) return;
  const int bh = u / units_per_head;
  const int ur = u - bh * units_per_head;
  int tiles[2];
  int ntiles = 1;
  // EXT: T query rows and S key rows per head; otherwise both are N
  const int Nq = EXT ? ex.T : N;
  const int Nk = EXT ? ex.S : N;
  if (CAUSAL && ex.pair) {
    tiles[0] = T_r - 1 - ur;  // heavy tile first
    tiles[1] = ur;
    ntiles = (tiles[1] < tiles[0]) ? 2 : 1;
  } else {
    tiles[0] = ur;
    tiles[1] = ur;
  }
  const bool split_mode = EXT && ex.nsplit > 1;
  int split = 0;
  if (split_mode) {
    split = ur % ex.nsplit;
    tiles[0] = tiles[1] = ur / ex.nsplit;
  }

  LaneOffsets<C> lo;
  lane_offsets<C>(lo, (unsigned)(uintptr_t)smem, w, lane);

  const size_t hoff = (size_t)bh * (size_t)Nq * C::D;
  // EXT: query head h of batch b reads K/V head h / group (the index is
  // wave-uniform; readfirstlane keeps the addresses derived from it scalar)
  size_t kvoff = hoff;
  if (EXT) {
    const unsigned kvh = (unsigned)__builtin_amdgcn_readfirstlane(
        (bh / ex.Hq) * (ex.Hq / ex.group) + (bh % ex.Hq) / ex.group);
    kvoff = (size_t)kvh * (size_t)Nk * C::D;
  }
  const uint16_t* qh = q + hoff;
  const uint16_t* kh = k + kvoff;
  const uint16_t* vh = v + kvoff;
  const int qoff = (EXT && CAUSAL) ? ex.offset : 0;   // position of query row 0
  const int wnd = (EXT && CAUSAL) ? ex.window : 0;    // sliding window (0: none)

  for (int ti = 0; ti < ntiles; ++ti) {
    // (EXT: said to be wave-uniform, so that the addresses derived from it
    // stay scalar)
    const int q0 = EXT ? __builtin_amdgcn_readfirstlane(tiles[ti] * C::BR) : tiles[ti] * C::BR;
    const int qw0 = q0 + w * 32;

    // Q_i rows as the B operand of S^T = K Q^T: lane holds query qw0 + l%32,
    // dims 16*kb + 8*(l/32) .. +7.  Rows past N are clamped (never stored).
    bf16x8 qr[C::KB];
    {
      const int row = min(qw0 + l32, Nq - 1);
      const uint16_t* src = qh + (size_t)row * C::D + 8 * h;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        u32x4 x = *(const u32x4*)(src + 16 * kb);
        x ^= qsign;  // exact sign flip when the caller's scale is negative
        qr[kb] = __builtin_bit_cast(bf16x8, x);
      }
    }

    int kv_end = CAUSAL ? min(Nk, qoff + q0 + C::BR) : Nk;
    // EXT with a window: the first key tile any query of the tile can see
    int kt0 = (EXT && wnd > 0) ? __builtin_amdgcn_readfirstlane(max(0, qoff + q0 - wnd + 1) / C::BC) : 0;
    if (split_mode) {  // this unit's chunk of keys
      kv_end = min(kv_end, (split + 1) * ex.chunk);
      kt0 = max(kt0, split * (ex.chunk / C::BC));
    }
    const int nkv = (kv_end + C::BC - 1) / C::BC - kt0;  // key tiles kt0 .. kt0 + nkv - 1
    // leading tiles that need no mask for any query of the workgroup
    int nfull = min(nkv, N / C::BC);
    if (CAUSAL) nfull = min(nfull, (q0 + 1) / C::BC);
    // tiles 1 .. jhead-1 are masked too (EXT: the window's left edge)
    int jhead = 1;
    if (EXT) {
      // unmasked: the tile lies below S and at or below every row's
      // position, and (window) after the tile holding the latest row's
      // first visible key, so that every row has set its reference before
      const int glast = min(Nk / C::BC, CAUSAL ? (qoff + q0 + 1) / C::BC : Nk / C::BC);
      const int gfirst = wnd > 0 ? max(0, qoff + q0 + C::BR - wnd) / C::BC + 1 : 1;
      nfull = max(0, min(nkv, glast - kt0));  // (split-KV: within the chunk)
      const int jh = max(1, gfirst - kt0);
      jhead = jh + ((1 - jh) & 3);  // the first j >= jh with j % 4 == 1 (unrolled stage order)
    }
    // Causal pairs: the light tile, run second, walks its key tiles from the
    // last to the first.  Every unit of a head then ends its light tile at
    // the same step, so the units read each key tile together (once from
    // HBM for all of them) instead of one after another from key 0 after
    // the tiles have left the L2.  The masked tiles (the diagonal, a ragged
    // end) then lead: tile j is key tile klast - j; the tiles from glast on,
    // which some row does not see in full, come first, plus tile glast - 1,
    // which every row sees, so that every row has set its reference (the
    // max of its first tile with a visible key) before the unmasked tiles.
    const bool desc = CAUSAL && ti == 1 && ex.pair;
    const int klast = kt0 + nkv - 1;
    if (desc) {
      const int glast = min(Nk / C::BC, (qoff + q0 + 1) / C::BC);
      const int jh = max(1, klast + 2 - glast);
      jhead = jh + ((1 - jh) & 3);
      nfull = nkv;
    }
    // key tile of step j (wave-uniform)
    auto ktile = [&](int j) __attribute__((always_inline)) { return desc ? klast - j : kt0 + j; };

    float m = -INFINITY;
    RowSums sums{0.f, 0.f};
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    // (split-KV: a chunk beyond every row's last visible key has no tiles)
    if (!EXT || nkv > 0) {
    // Phases.  Each step j of a wave is a matrix-core phase M(j) -- S_j =
    // K_j Q^T and acc += V_{j-1}^T P_{j-1}^T -- followed by a vector-ALU
    // phase V(j) -- the softmax of S_j into P_j -- with a workgroup barrier
    // after every phase.  Waves w and w + 4 share a SIMD; waves 4..7 run one
    // phase behind waves 0..3 (one extra barrier at the start, one fewer at
    // the end), so on every SIMD one wave feeds the matrix cores while the
    // other computes exponentials; the matrix phase runs at raised wave
    // priority so that its MFMAs issue first.
    // K and V tiles rotate through NST = 4 LDS stages each (tile t in stage
    // t % 4); waves 0..3 copy K, waves 4..7 copy V.  Number the barriers so
    // that the leading half's M(j) ends at barrier 2j+2 (the lagging half's
    // at 2j+3).  K_t is last read in the lagging M(t) (ends 2t+3), V_t in the
    // lagging M(t+1) (ends 2t+5).
    //  VCOPY: V(j) also issues this wave's copies for tile j+3, waits for its
    //   copies of tile j+2, and reads ahead the first K operands of tile
    //   j+1.  The leading half writes K_{t+4} from barrier 2t+4 on, the
    //   lagging half V_{t+4} from 2t+5 on: after the last reads of the
    //   stage; both waits end by barrier 2t+8, before tile t+4 is first read
    //   (the read-ahead in the leading V(t+3)).
    //  !VCOPY: M(j) starts with this wave's copies for tile j+2 and ends
    //   with the wait for its copies of tile j+1.  K_{t+4} is written from
    //   barrier 2t+5 (leading M(t+2)), V_{t+4} from 2t+6; K_{t+4} has landed
    //   by 2t+8 (end of the leading M(t+3)) and V_{t+4} by 2t+9, before their
    //   first reads (leading M(t+4) from 2t+9, and its P V in M(t+5)).
    constexpr bool VC = C::VCOPY;
    constexpr int AHEAD = VC ? 3 : 2;  // copies run this many tiles ahead
    const bool lag = w >= C::NCW;
    const uint16_t* msrc = lag ? vh : kh;                     // the matrix this wave copies
    const unsigned mdst = lo.base + (lag ? C::VBASE : 0u);  // ... and its LDS ring
    f32x16 s[C::SB];
    bf16x8 p[C::PB];  // P_{j-1} is read in M(j), then P_j is written in V(j)
    // (two-barrier schedule: V(j) leaves P_j unpacked in s; M(j+1) packs it)
    PendingP pend{0.f, false};
    bf16x8 kpre[C::KD][C::SB];
    // S_j = K_j Q^T once more, from the K tile at stage offset kst (still in
    // LDS during the vector phase of step j): the rare path of tile_softmax
    auto rescore_at = [&](int kst) __attribute__((always_inline)) {
      const f32x16 zero = {};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb)
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_k<C>(lo, kst, kb, sb), qr[kb], kb == 0 ? zero : s[sb],
                                                          0, 0, 0);
    };
    // M(j) (HAS_QK: K_j at stage offset kst; HAS_PV: V_{j-1} at vst); !VCOPY:
    // copies for tile j+2 into stage offset dst
    auto mphase = [&](int j, int kst, int vst, int dst, auto has_qk, auto has_pv) __attribute__((always_inline)) {
      constexpr bool QK = decltype(has_qk)::value, PV = decltype(has_pv)::value;
      if (!VC) {
        if (j + 2 < nkv) load_tile<C>(msrc, mdst + dst, ktile(j + 2) * C::BC, Nk, lo, w);
        if (QK) prefetch_k<C>(kpre, lo, kst);
      }
      tile_m<C, QK, PV, !VC>(kst, vst, lo, qr, s, p, acc, kpre, sums, pend);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) pin(acc[db]);
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) pin(s[sb]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if (!VC) {
        if (j + 2 < nkv) wait_copies<C::NI>();
        else wait_copies<0>();
      }
    };
    // V(j): softmax of tile j; VCOPY: copies for tile j+3 into stage offset
    // dst, then read ahead K of tile j+1 at stage offset kst1
    auto vphase = [&](int j, int kst0, int dst, int kst1, auto mask_tag, auto first_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr bool FIRST = decltype(first_tag)::value;
      tile_softmax<C, CAUSAL, MASK, FIRST, VC>(s, p, acc, m, sums, pend, ktile(j) * C::BC, qoff + qw0, Nk, c,
                                               lane, wnd, [&]() __attribute__((always_inline)) { rescore_at(kst0); });
      __builtin_amdgcn_sched_barrier(0);
      if (VC) {
        if (j + 3 < nkv) {
          load_tile<C>(msrc, mdst + dst, ktile(j + 3) * C::BC, Nk, lo, w);
          wait_copies<C::NI>();
        } else {
          wait_copies<0>();
        }
        if (j + 1 < nkv) prefetch_k<C>(kpre, lo, kst1);
      }
      barrier();
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    };
    // one step; stages of tiles j, j-1, j+AHEAD, j+1 (compile-time constants
    // in the unrolled loop, run-time values otherwise)
    auto step = [&](int j, int kst, int vst, int dst, int kst1, auto mask_tag) __attribute__((always_inline)) {
      mphase(j, kst, vst, dst, std::true_type{}, std::true_type{});
      barrier();
      vphase(j, kst, dst, kst1, mask_tag, std::false_type{});
    };
    constexpr int KT = C::KT;
    auto stg = [](int t) __attribute__((always_inline)) { return (t & 3) * KT; };

    if constexpr (VC) {
      // One barrier per step.  Between barriers j and j+1 (window j) the
      // leading half runs V(j) then M(j+1), the lagging half M(j) then V(j):
      // each SIMD still alternates a matrix phase of one wave with the
      // vector phase of the other, with half the synchronisation.  In window
      // j the leading half copies K_{j+3} (into the stage of K_{j-1}, whose
      // last reads were in window j-1) and waits for K_{j+2}; the lagging
      // half copies V_{j+2} (stage of V_{j-2}, last read in window j-1) and
      // waits for V_{j+1}.  So K_t and V_t are complete by barrier t-1, and
      // the first reads of tile t -- the read-ahead of K_t in window t-1 and
      // the leading P V of tile t in window t+1 -- come after it.
      auto m1 = [&](int kst, int vst, auto has_qk, auto has_pv) __attribute__((always_inline)) {
        constexpr bool QK = decltype(has_qk)::value, PV = decltype(has_pv)::value;
        tile_m<C, QK, PV>(kst, vst, lo, qr, s, p, acc, kpre, sums, pend);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) pin(acc[db]);
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) pin(s[sb]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      // V(j) with the stages of tiles j, j+1, j+2, j+3 (LAG: this wave is in
      // the lagging half, which copies V; the leading half copies K)
      auto v1 = [&](int j, int s0, int s1, int s2, int s3, auto lag_tag, auto mask_tag, auto first_tag) __attribute__((always_inline)) {
        constexpr bool LAG = decltype(lag_tag)::value;
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr bool FIRST = decltype(first_tag)::value;
        tile_softmax<C, CAUSAL, MASK, FIRST, true>(s, p, acc, m, sums, pend, ktile(j) * C::BC, qoff + qw0, Nk, c,
                                                   lane, wnd, [&]() __attribute__((always_inline)) { rescore_at(s0); });
        __builtin_amdgcn_sched_barrier(0);
        const int ct = LAG ? j + 2 : j + 3;  // the tile this wave copies now
        if (ct < nkv) {
          load_tile<C>(LAG ? vh : kh, lo.base + (LAG ? C::VBASE + s2 : s3), ktile(ct) * C::BC, Nk, lo, w);
          wait_copies<C::NI>();
        } else {
          wait_copies<0>();
        }
        if (j + 1 < nkv) prefetch_k<C>(kpre, lo, s1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
      };
      // the whole key loop of one half (each half gets its own copy of the
      // code, so that the register allocation follows its own phase order)
      auto run = [&](auto lag_tag) __attribute__((always_inline)) {
        constexpr bool LAG = decltype(lag_tag)::value;
        const std::true_type T{};
        const std::false_type F{};
        // window j for 1 <= j < nkv - 1, stages of tiles j-1 .. j+3
        auto window = [&](int j, int sm1, int s0, int s1, int s2, int s3, auto mask_tag) __attribute__((always_inline)) {
          if (!LAG) {
            v1(j, s0, s1, s2, s3, lag_tag, mask_tag, F);
            m1(s1, s0, T, T);
          } else {
            m1(s0, sm1, T, T);
            v1(j, s0, s1, s2, s3, lag_tag, mask_tag, F);
          }
          barrier();
        };
        for (int t = 0; t < (LAG ? 2 : 3); ++t)
          if (t < nkv)
            load_tile<C>(LAG ? vh : kh, lo.base + (LAG ? C::VBASE : 0) + stg(t), ktile(t) * C::BC, Nk, lo, w);
        wait_copies<0>();
        barrier();
        prefetch_k<C>(kpre, lo, 0);
        __builtin_amdgcn_s_setprio(1);
        if (!LAG) m1(0, 0, T, F);  // leading M(0)
        barrier();
        // window 0 (its tile may need the mask: the mask is exact on any tile)
        if (!LAG) {
          v1(0, stg(0), stg(1), stg(2), stg(3), lag_tag, T, T);
          if (1 < nkv) m1(stg(1), stg(0), T, T);
          else m1(0, stg(0), F, T);
        } else {
          m1(0, 0, T, F);
          v1(0, stg(0), stg(1), stg(2), stg(3), lag_tag, T, T);
        }
        barrier();
        // unmasked windows 1 .. j1-1, unrolled by the ring size so that
        // every stage offset is a compile-time constant
        const int j1 = max(1, min(nfull, nkv - 1));
        int j = 1;
        for (; j < min(jhead, j1); ++j) window(j, stg(j - 1), stg(j), stg(j + 1), stg(j + 2), stg(j + 3), T);
        for (; j + 3 < j1; j += 4) {
          window(j + 0, stg(0), stg(1), stg(2), stg(3), stg(4), F);
          window(j + 1, stg(1), stg(2), stg(3), stg(4), stg(5), F);
          window(j + 2, stg(2), stg(3), stg(4), stg(5), stg(6), F);
          window(j + 3, stg(3), stg(4), stg(5), stg(6), stg(7), F);
        }
        if (j < j1) { window(j, stg(0), stg(1), stg(2), stg(3), stg(4), F); ++j; }
        if (j < j1) { window(j, stg(1), stg(2), stg(3), stg(4), stg(5), F); ++j; }
        if (j < j1) { window(j, stg(2), stg(3), stg(4), stg(5), stg(6), F); ++j; }
        // masked windows up to nkv - 2, stages at run time
        for (; j < nkv - 1; ++j) window(j, stg(j - 1), stg(j), stg(j + 1), stg(j + 2), stg(j + 3), T);
        // the last window (nkv >= 2): the leading half's M(nkv) is P V only
        if (nkv >= 2) {
          const int jl = nkv - 1;
          if (!LAG) {
            v1(jl, stg(jl), stg(jl + 1), stg(jl + 2), stg(jl + 3), lag_tag, T, F);
            m1(0, stg(jl), F, T);
          } else {
            m1(stg(jl), stg(jl - 1), T, T);
            v1(jl, stg(jl), stg(jl + 1), stg(jl + 2), stg(jl + 3), lag_tag, T, F);
          }
          barrier();
        }
        // the lagging half's M(nkv): the last P V
        if (LAG) m1(0, stg(nkv - 1), F, T);
      };
      if (lag) run(std::true_type{});
      else run(std::false_type{});
      barrier();  // every wave is done with the LDS ring before it is refilled
    } else {

      for (int t = 0; t < AHEAD; ++t)
        if (t < nkv) load_tile<C>(msrc, mdst + stg(t), ktile(t) * C::BC, Nk, lo, w);
      wait_copies<0>();
      barrier();
      if (lag) barrier();
      __builtin_amdgcn_s_setprio(1);
      // M(0), V(0)
      if (VC) prefetch_k<C>(kpre, lo, 0);
      mphase(0, 0, 0, stg(AHEAD), std::true_type{}, std::false_type{});
      barrier();
      // (EXT: the first tile may be the window's left edge: always masked)
      if (nfull > 0 && !EXT && !desc) vphase(0, 0, stg(AHEAD), stg(1), std::false_type{}, std::true_type{});
      else vphase(0, 0, stg(AHEAD), stg(1), std::true_type{}, std::true_type{});
      // unmasked steps 1 .. j1-1, unrolled by the ring size so that every
      // stage offset is a compile-time constant (step j uses stage j % 4)
      const int j1 = max(1, min(nfull, nkv));
      int j = 1;
      for (; j < min(jhead, j1); ++j)
        step(j, stg(j), stg(j - 1), stg(j + AHEAD), stg(j + 1), std::true_type{});
      for (; j + 3 < j1; j += 4) {
        step(j + 0, stg(1), stg(0), stg(1 + AHEAD), stg(2), std::false_type{});
        step(j + 1, stg(2), stg(1), stg(2 + AHEAD), stg(3), std::false_type{});
        step(j + 2, stg(3), stg(2), stg(3 + AHEAD), stg(4), std::false_type{});
        step(j + 3, stg(4), stg(3), stg(4 + AHEAD), stg(5), std::false_type{});
      }
      if (j < j1) { step(j, stg(1), stg(0), stg(1 + AHEAD), stg(2), std::false_type{}); ++j; }
      if (j < j1) { step(j, stg(2), stg(1), stg(2 + AHEAD), stg(3), std::false_type{}); ++j; }
      if (j < j1) { step(j, stg(3), stg(2), stg(3 + AHEAD), stg(4), std::false_type{}); ++j; }
      // remaining (masked) steps, stages at run time
      for (; j < nkv; ++j) step(j, stg(j), stg(j - 1), stg(j + AHEAD), stg(j + 1), std::true_type{});
      // M(nkv): the last P V
      mphase(nkv, 0, stg(nkv - 1), 0, std::false_type{}, std::true_type{});
      if (!lag) barrier();
      barrier();  // every wave is done with the LDS ring before it is refilled
    }

    }

    // ---- epilogue: O = acc / l (bf16, RNE), LSE = (m + log2 l) * ln 2
    const float lt = 2.f * half_sum(sums.lh);
    const float ltb = lt + half_sum(sums.corr);
    // (split-KV: no visible key in this chunk -> O_g = 0, LSE_g = -inf)
    const bool empty = EXT && !(lt > 0.f);
    const float inv = empty ? 0.f : 1.f / ltb;
    const int query = qw0 + l32;
    if (split_mode && query < Nq) {
      const size_t prow = ((size_t)split * ex.BH + bh) * Nq + query;
      float* orow = ex.ws_o + prow * C::D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float4 ov;
          ov.x = acc[db][4 * a + 0] * inv;
          ov.y = acc[db][4 * a + 1] * inv;
          ov.z = acc[db][4 * a + 2] * inv;
          ov.w = acc[db][4 * a + 3] * inv;
          *(float4*)(orow + 32 * db + 8 * a + 4 * h) = ov;
        }
      if (h == 0) ex.ws_lse[prow] = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
    } else if (!split_mode) {
      // O (bf16, RNE) through this wave's LDS staging area: row-major with
      // the 16-byte chunks of row r XOR-swizzled by (r / rows per 256 bytes)
      // so that the 8-byte writes spread over the banks; read back as whole
      // rows, 64 lanes x 16 bytes (1 KB, 256 / ROWB * 4 rows) per store.
      // Only this wave reads what it wrote, so no barrier is needed.
      constexpr int CPR = C::CPR;               // 16-byte chunks per row
      constexpr int RP2 = 256 / C::ROWB;        // rows per 256 bytes (1 or 2)
      // (the lane index is made opaque so that these addresses are computed
      // here, not hoisted out of the query-tile loop into live registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      unsigned char LDS_AS* stg_o = smem + C::OBASE + w * C::OROWS;
      const int r0 = ln & 31, sw = (r0 / RP2) & (CPR - 1);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[db][4 * a + e] * inv);
          *(u32x2 LDS_AS*)(stg_o + r0 * C::ROWB + 16 * ((4 * db + a) ^ sw) + 8 * (ln >> 5)) =
              __builtin_bit_cast(u32x2, ov);
        }
      constexpr int RPS = 64 / CPR;             // rows per store instruction
#pragma unroll
      for (int i = 0; i < 32 / RPS; ++i) {
        const int r = i * RPS + ln / CPR;       // row within the wave's 32
        const int ch = ln % CPR;
        const u32x4 x = *(const u32x4 LDS_AS*)(stg_o + r * C::ROWB + 16 * (ch ^ ((r / RP2) & (CPR - 1))));
        if (qw0 + r < Nq) *(u32x4*)(o + hoff + (size_t)(qw0 + r) * C::D + 8 * ch) = x;
      }
      if (h == 0 && query < Nq) lse[(size_t)bh * Nq + query] = (m + __log2f(lt)) * kLn2;
    }
  }
}

// The forward kernel: one work unit per workgroup.
template <class C, bool CAUSAL, bool EXT = false>
__global__ void __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
                   int N, int T_r, int units_per_head, int num_units, int per_xcd, float c,
                   unsigned int qsign, ExtArgs ex) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_TOTAL];
  fwd_unit<C, CAUSAL, EXT>(q, k, v, o, lse, N, T_r, units_per_head, num_units, per_xcd, c, qsign, ex,
                           (unsigned char LDS_AS*)smem);
}

// ---------------------------------------------------------------------------
// Host side.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
          int N, int d, float scale, int elem_bytes) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const long long rows = (long long)B * H * N;
  if (rows == 0) return FA_OK;
  if ((long long)B * H > (1LL << 30) || rows > (1LL << 40)) return FA_ERR_SHAPE;
  // grid size: query tiles of at least 32 rows per (b, h), padded to 8
  if ((long long)B * H * ((N + 31) / 32) > (1LL << 30)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  const size_t nb = (size_t)rows * d * elem_bytes;
  const size_t lb = (size_t)rows * sizeof(float);
  if (overlaps(o, nb, q, nb) || overlaps(o, nb, k, nb) || overlaps(o, nb, v, nb) ||
      overlaps(lse, lb, q, nb) || overlaps(lse, lb, k, nb) || overlaps(lse, lb, v, nb) ||
      overlaps(lse, lb, o, nb))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Causal work units pair the heavy query tile T_r-1-u with the light tile u,
// so that every unit costs about the same -- when there are more query
// tiles than compute units.  With fewer, every tile gets a compute unit of
// its own: the call then takes as long as its heaviest tile, not as long as
// the heaviest pair on half of the chip.
constexpr long long kComputeUnits = 256;  // MI355X
inline bool pair_tiles(long long heads, int T_r) { return heads * T_r > kComputeUnits; }

template <class C, bool CAUSAL>
void launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                 float c, unsigned qsign, hipStream_t stream) {
  const int T_r = (N + C::BR - 1) / C::BR;
  const int pair = CAUSAL && pair_tiles((long long)B * H, T_r);
  const int units_per_head = pair ? (T_r + 1) / 2 : T_r;
  const int num_units = B * H * units_per_head;
  const int per_xcd = (num_units + 7) / 8;
  const int grid = per_xcd * 8;
  ExtArgs ex{};
  ex.pair = pair;
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<C, CAUSAL>), dim3(grid), dim3(C::NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, N, T_r,
                     units_per_head, num_units, per_xcd, c, qsign, ex);
}

template <class C, bool CAUSAL>
void launch_bf16_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                    int T, int S, int offset, int window, float c, unsigned qsign, hipStream_t stream,
                    int nsplit = 1, int chunk = 0, float* ws_o = nullptr, float* ws_lse = nullptr) {
  const int T_r = (T + C::BR - 1) / C::BR;
  // with a window (or split keys) every unit costs about the same: no pairing
  const int pair = CAUSAL && window == 0 && nsplit == 1 && pair_tiles((long long)B * Hq, T_r);
  const int units_per_head = pair ? (T_r + 1) / 2 : T_r * nsplit;
  const int num_units = B * Hq * units_per_head;
  const int per_xcd = (num_units + 7) / 8;
  const int grid = per_xcd * 8;
  const ExtArgs ex{T, S, Hq, Hq / Hkv, offset, window, pair, nsplit, chunk, B * Hq, ws_o, ws_lse};
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<C, CAUSAL, true>), dim3(grid), dim3(C::NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, T, T_r,
                     units_per_head, num_units, per_xcd, c, qsign, ex);
}

int check_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
             int Hkv, int T, int S, int d, float scale, int causal, int offset, int window) {
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0 || S < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const long long rows = (long long)B * Hq * T;
  if (rows == 0) return FA_OK;
  if (Hkv == 0 || Hq % Hkv != 0) return FA_ERR_VARIANT;
  if (S == 0) return FA_ERR_VARIANT;  // a query row would see no key
  if (window < 0 || (window > 0 && !causal)) return FA_ERR_VARIANT;
  if (causal && (offset < 0 || offset > S - T)) return FA_ERR_VARIANT;
  const long long krows = (long long)B * Hkv * S;
  if ((long long)B * Hq > (1LL << 30) || rows > (1LL << 40) || krows > (1LL << 40)) return FA_ERR_SHAPE;
  if ((long long)B * Hq * ((T + 31) / 32) > (1LL << 30)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  const size_t qb = (size_t)rows * d * 2;
  const size_t kb = (size_t)krows * d * 2;
  const size_t lb = (size_t)rows * sizeof(float);
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) || overlaps(lse, lb, q, qb) ||
      overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) || overlaps(lse, lb, o, qb))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Tile shapes (B_c keys per K/V tile, NW waves of 32 query rows: B_r = 32 NW).
// The defaults are the library's; other values build the variants that the
// tile-size sweep measures (where the LDS ring, the registers and the copy
// mapping allow them: the static_asserts of Cfg).
#ifndef FA_D128_BC
#define FA_D128_BC 64
#endif
#ifndef FA_D64_BC
#define FA_D64_BC 128
#endif
#ifndef FA_D128_NW
#define FA_D128_NW 8
#endif
#ifndef FA_D64_NW
#define FA_D64_NW 8
#endif
using CfgD128 = Cfg<128, FA_D128_BC, FA_D128_NW>;
using CfgD64 = Cfg<64, FA_D64_BC, FA_D64_NW>;

}  // namespace

namespace fa {

bool host_overlaps(const void* a, size_t na, const void* b, size_t nb) { return overlaps(a, na, b, nb); }

int host_check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int N,
               int d, float scale, int elem_bytes) {
  return check(q, k, v, o, lse, B, H, N, d, scale, elem_bytes);
}

int host_check_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
                  int Hkv, int T, int S, int d, float scale, int causal, int offset, int window) {
  return check_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window);
}

void host_launch_ex_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                          int T, int S, int d, int causal, int offset, int window, float c, unsigned qsign,
                          int nsplit, int chunk, float* ws_o, float* ws_lse, hipStream_t stream) {
  if (d == 128) {
    if (causal)
      launch_bf16_ex<CfgD128, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, offset, window, c, qsign, stream, nsplit,
                                    chunk, ws_o, ws_lse);
    else
      launch_bf16_ex<CfgD128, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, offset, window, c, qsign, stream, nsplit,
                                     chunk, ws_o, ws_lse);
  } else {
    if (causal)
      launch_bf16_ex<CfgD64, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, offset, window, c, qsign, stream, nsplit,
                                   chunk, ws_o, ws_lse);
    else
      launch_bf16_ex<CfgD64, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, offset, window, c, qsign, stream, nsplit,
                                    chunk, ws_o, ws_lse);
  }
}

}  // namespace fa

extern "C" int fa_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             int B, int H, int N, int d, float scale, int causal, int elem_bytes) {
  (void)causal;
  if (elem_bytes != 2 && elem_bytes != 4) return FA_ERR_SHAPE;
  return check(q, k, v, o, lse, B, H, N, d, scale, elem_bytes);
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                      int d, float scale, int causal, hipStream_t stream) {
  const int st = check(q, k, v, o, lse, B, H, N, d, scale, 2);
  if (st != FA_OK) return st;
  if ((long long)B * H * N == 0) return FA_OK;
  // Scores are formed as |scale| * (sign(scale) Q) K^T: a negative scale flips
  // the sign bit of every Q element (exact), so the kernel sees c >= 0.
  const unsigned qsign = (scale < 0.f) ? 0x80008000u : 0u;
  // A zero scale runs as 2^-100: every visible weight exp2(s * 2^-100 - m)
  // then rounds to exactly 1 in fp32 (for |s| < 2^75), i.e. the plain mean
  // of the visible V rows, while masked scores still map to exp2(-inf) = 0.
  const float c = scale == 0.f ? 0x1p-100f : fabsf(scale) * kLog2e;
  if (d == 128) {
    if (causal) launch_bf16<CfgD128, true>(q, k, v, o, lse, B, H, N, c, qsign, stream);
    else launch_bf16<CfgD128, false>(q, k, v, o, lse, B, H, N, c, qsign, stream);
  } else {
    if (causal) launch_bf16<CfgD64, true>(q, k, v, o, lse, B, H, N, c, qsign, stream);
    else launch_bf16<CfgD64, false>(q, k, v, o, lse, B, H, N, c, qsign, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_check_args_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                int B, int Hq, int Hkv, int T, int S, int d, float scale, int causal, int offset,
                                int window) {
  return check_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window);
}

extern "C" int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int T, int S, int d, float scale, int causal, int offset, int window,
                         hipStream_t stream) {
  const int st = check_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, offset, window);
  if (st != FA_OK) return st;
  if ((long long)B * Hq * T == 0) return FA_OK;
  const unsigned qsign = (scale < 0.f) ? 0x80008000u : 0u;  // as in fa_fwd
  const float c = scale == 0.f ? 0x1p-100f : fabsf(scale) * kLog2e;
  const int off = causal ? offset : 0;
  const int wnd = causal ? window : 0;
  if (d == 128) {
    if (causal) launch_bf16_ex<CfgD128, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, off, wnd, c, qsign, stream);
    else launch_bf16_ex<CfgD128, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, off, wnd, c, qsign, stream);
  } else {
    if (causal) launch_bf16_ex<CfgD64, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, off, wnd, c, qsign, stream);
    else launch_bf16_ex<CfgD64, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, off, wnd, c, qsign, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_supported(int d, int dtype) {
  return (d == 64 || d == 128) && (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F32) ? 1 : 0;
}

extern "C" const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid or too large shape (B, H, N)";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension (need 64 or 128)";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIAS: return "output buffers overlap inputs or each other";
    case FA_ERR_LAUNCH: return "HIP kernel launch failed";
    case FA_ERR_ALIGN: return "pointer not aligned (16 bytes for q/k/v/o, 4 for lse)";
    case FA_ERR_VARIANT: return "inconsistent heads, offset or window (fa_fwd_ex)";
    case FA_ERR_SCRATCH: return "partials larger than the static scratch (fa_fwd_split_noalloc)";
    default: return "unknown status";
  }
}
