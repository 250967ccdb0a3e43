// av_fwd_kernel.h — forward kernel: exact attention over packed variable-length
// sequences with grouped-query heads, bf16 in, fp32 accumulation, optional LSE.
// Instantiated by av_fwd.hip (one pass over every visible key) and
// av_fwd_split.hip (the keys of an item split over several workgroups).
//
// What it computes follows the forward loop the FlashAttention repository guide
// describes under Key Patterns (load a Q tile, loop over K/V blocks, online
// softmax with running row max and row sum, store O and LSE) and Core
// Abstractions (online softmax; causal block ranges; varlen offsets). The
// result is the exact softmax(QK^T * scale + mask) V of each packed sequence.
//
// gfx950 design (one workgroup = BM / 32 waves sharing every K / V tile; each
// wave owns 32 query rows of one query head; the waves cover hw heads of one
// KV group and BM / hw rows of each, hw = block_heads(group size)):
//  * Q^T stays in VGPRs for the whole item as the B operand of S^T = K Q^T.
//  * K and V tiles of 64 keys go HBM -> LDS with buffer_load ... lds (no VGPR
//    staging, out-of-range rows read as zero) into separate double buffers.
//    Rows are stored row-major with an XOR swizzle of 16-byte chunks (swz<D>).
//    The tile's first row is folded into the buffer descriptor (scalar ops),
//    so the per-lane copy offsets never change.
//  * Software pipeline inside each wave. Iteration n holds the scores of tile
//    n and runs two phases: (B) the MFMAs of S(n+1) = K(n+1) Q^T interleaved
//    with the exp / row-sum / bf16 packing of most of P(n); (C) the MFMAs of
//    O^T += V(n)^T P(n)^T interleaved with the rest of P(n) and the row max of
//    S(n+1). The vector ALU work of the softmax thus issues while the matrix
//    cores run, instead of between MFMA bursts. K(n+1) and V(n) are resident
//    together, and the copies of K(n+2) and V(n+1) are in flight meanwhile.
//  * V^T comes from the row-major V tile through transposing LDS reads
//    (ds_read_b64_tr_b16); the key permutation kperm makes the fp32 score
//    registers the B operand of the PV product after a bf16 conversion.
//  * Each lane owns one query column: running max, running sum and rescale
//    factor are per-lane values; the row max needs one exchange with lane ^ 32
//    per tile (v_permlane32_swap), the row sum is combined once at the end.
//  * exp2 with the scale folded into one FMA per score. The running max is
//    only moved (and O rescaled) when a tile's max exceeds it by more than
//    kRescaleSlack (in log2 units), so P <= 2^kRescaleSlack and most tiles do
//    no rescaling; the result is the same softmax, only the reference point of
//    the exponentials changes. Two row sums are kept: the fp32 sum of P gives
//    the LSE, and the sum of the bf16-rounded P that enter the PV product
//    normalises O, so the rounding of P cancels in O's weighted average even
//    when one key carries almost all of a row's weight.
//  * Masking runs only on key tiles that cross the causal diagonal or the end
//    of the sequence: their invisible scores are set to -inf once, when the
//    tile's scores are formed (the scale factor is always > 0, so exp2 maps
//    them to exactly 0). Tiles past the causal range are never visited. On
//    masked tiles P is split into bf16 hi + lo parts so rows with very few
//    visible keys stay accurate.
#ifndef AV_FWD_KERNEL_H
#define AV_FWD_KERNEL_H

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "av_common.h"
#include "av_exp2.h"
#include "av_launch.h"
#include "av_tiles.h"

namespace av {

constexpr float kRescaleSlack = 8.0f;

template <int D, int BM_, int BN_>
struct FwdCfg {
  using KV = RowTile<D, BN_>;
  static constexpr int BM = BM_;                      // query rows per workgroup
  static constexpr int WAVES = BM / 32;               // one wave per 32 rows
  static constexpr int BN = BN_;                      // keys per tile (32 or 64)
  static constexpr int NA = BN / 32;                  // 32-key score accumulators per wave
  static constexpr int NS = BN / 2;                   // scores per lane per tile
  static constexpr int NJ = BN / 16;                  // 16-key k-steps of the PV product
  static constexpr int NT = 64 * WAVES;               // threads per workgroup
  static constexpr int ROW = KV::ROW;                 // bytes per key row in LDS
  static constexpr int TILE = KV::BYTES;              // bytes of one K or V tile
  static constexpr int VBASE = 2 * TILE;              // K0 K1 | V0 V1
  static constexpr size_t LDS_BYTES = 4 * TILE;
  static constexpr int DMA = KV::DMAS / WAVES;        // copies per wave per tile
  static constexpr int KK = D / 16;                   // k-steps of S = K Q^T
  static constexpr int DB = D / 32;                   // 32-wide head-dim blocks of O
  static constexpr int PF = 2;                        // K operand prefetch distance
  // head_dim 256 needs more than 256 registers per lane (O alone is 128): one
  // wave per SIMD, with the accumulators free to use AGPRs
  static constexpr int WAVES_PER_SIMD = (D <= 128) ? 2 : 1;
  static constexpr int MIN_BLOCKS_PER_CU = WAVES_PER_SIMD * 4 / WAVES;
  static_assert(KV::DMAS % WAVES == 0, "tile copies must split evenly over the waves");
  static_assert(LDS_BYTES * MIN_BLOCKS_PER_CU <= 160 * 1024, "LDS budget");
};

// The forward kernel's tile sizes for a head_dim (the grid depends on BM).
// head_dim 256 uses 32-key tiles: the four K / V buffers then take 64 KB, so
// every LDS operand address is a register plus a 16-bit immediate, and the
// score state of the pipeline halves.
template <int D>
struct FwdBlock {
  static constexpr int BM = 128;
  static constexpr int BN = (D <= 128) ? 64 : 32;
  static_assert(BM == kQueryBlock && BN == key_tile(D), "tile shapes of the host-side plan");
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* out;
  float* lse;
  int num_seqs;
  int total_q;
  int Hq;
  int Hkv;
  // A workgroup's waves cover hw query heads of one KV group (hw divides both
  // the group size and the wave count) and, for each, bm = 32 waves / hw query
  // rows; hw_log2 = log2(hw). With hw > 1 the causal diagonal of a block
  // crosses fewer key tiles.
  int hw, hw_log2, bm;
  int levels;        // ceil(max_seqlen_q / bm)
  float scale_log2;  // |softmax_scale| * log2(e), at least FLT_MIN
  int neg_scale;     // softmax_scale < 0: Q is negated so the scale is positive
  int wl, wr;        // visible band of a row (keys i + Lk - Lq - wl .. + wr; < 0: unbounded)
  // split-KV partial results (SPLIT kernels only): the item's key tiles are cut
  // into `splits` contiguous chunks, one workgroup each; chunk s writes its O,
  // normalised over its own keys, as fp32 part_o[s][total_q][Hq][D], and its two
  // log2-domain row sums part_l[s][0 / 1][Hq][total_q] (sum of P, sum of the
  // bf16-rounded P; -inf when the chunk holds no visible key of the row)
  float* part_o;
  float* part_l;
  int splits;
  // persistent scheduling (fwd_kernel_persistent only): 8 queue counters and a
  // count of finished workgroups, all 0 on entry and returned to 0 on exit
  unsigned int* sched;
};

// O^T accumulation. At head_dim 256 (one wave per SIMD, O = 128 registers per
// lane) the accumulators are pinned to AGPRs: an empty asm statement with an
// AGPR operand follows every MFMA (left to itself the register allocator gives
// the loop-carried O different register files in the two unrolled steps and
// copies all of it every step). The MFMA itself stays the compiler's builtin:
// the allocator still inserts some AGPR-to-AGPR copies of O where control flow
// joins, and only an MFMA the compiler can see gets the wait states such a copy
// needs before it reads the result (an MFMA written in asm does not, and the
// last registers of its result were then read stale). o_fence() keeps the
// VALU passes over O (rescale, epilogue) in their place.
template <int D>
__device__ __forceinline__ void pv_mfma(f32x16& o, const bf16x8& v, const bf16x8& p) {
  o = mfma32x32x16(v, p, o);
  if constexpr (D == 256) asm volatile("" : "+a"(o));
}

template <int D, int DB>
__device__ __forceinline__ void o_fence(f32x16 (&o)[DB]) {
  if constexpr (D == 256) {
    static_assert(DB == 8, "fence written for 8 accumulators");
    asm volatile("" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
  }
}

// Descriptor of the same rows starting `bytes` further on.
__device__ __forceinline__ i32x4 rsrc_advance(const i32x4& r, uint32_t bytes) {
  const uint64_t base = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + bytes;
  i32x4 o;
  o[0] = (int)(uint32_t)base;
  o[1] = (int)((uint32_t)(base >> 32) & 0xffffu);
  o[2] = (int)((uint32_t)r[2] - bytes);
  o[3] = r[3];
  return o;
}

// Per-wave state of the forward item that the pipeline steps share.
template <int D, int BM, int BN, int MODE>
struct FwdCtx {
  using T = FwdCfg<D, BM, BN>;
  static constexpr bool LEFT = MODE == 2;  // rows' bands have a first key (a left window bound)
  const lds_char* lds;
  uint32_t lds0;
  i32x4 rk, rv;          // K / V rows of this (sequence, KV head), from key 0
  uint32_t tile_bytes;   // BN rows of the K / V tensor
  // This lane's source offset within a tile: per copy, or (ONE_VOFF) for the
  // first copy only, the others being whole rounds of rows further on. The
  // latter costs an add per copy but frees registers: it is used where the
  // kernel would otherwise spill (banded masks at head_dim 64 / 128).
  static constexpr bool ONE_VOFF = D <= 128 && MODE >= 1;
  uint32_t voff[ONE_VOFF ? 1 : T::DMA];
  uint32_t round_bytes;  // ONE_VOFF: rows copied by all waves' i-th copies
  int wave, half;
  int ntiles;            // one past the item's last tile
  int kvis_lo;           // first key visible to this lane's query row
  int kvis_end;          // one past the last one
  float c;               // exp2 scale factor
  OperandOffsets<D> off;
  bf16x8 qf[T::KK];
};

// Copy this wave's share of a tile (rows row0 ..) into LDS at `dst`. With
// ONE_VOFF, copy i of wave w is the tile's copy i * WAVES + w: at head_dim 64
// and 128 the chunk swizzle of its rows is then the same for every i, so the
// source offsets of a lane differ by whole rounds of rows, added here (behind an
// empty asm statement, so that the sums are not hoisted and held in registers).
template <int D, int BM, int BN, int MODE>
__device__ __forceinline__ void issue_tile(const FwdCtx<D, BM, BN, MODE>& x, uint32_t dst, const i32x4& rsrc, int row0) {
  using T = FwdCfg<D, BM, BN>;
  const i32x4 r = rsrc_advance(rsrc, (uint32_t)row0 * (x.tile_bytes / T::BN));
  if constexpr (FwdCtx<D, BM, BN, MODE>::ONE_VOFF) {
    uint32_t v = x.voff[0];
    asm volatile("" : "+v"(v));
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) lds_dma16(r, dst + (i * T::WAVES + x.wave) * 1024, v + i * x.round_bytes);
  } else {
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) lds_dma16(r, dst + (x.wave * T::DMA + i) * 1024, x.voff[i]);
  }
}

// Score register v of accumulator a (a = 0: keys 0..31 of the tile, a = 1:
// keys 32..63) is key 32 a + 16 (v / 8) + 8 half + v % 8.
template <int D, int BM, int BN, int MODE>
__device__ __forceinline__ void mask_scores(const FwdCtx<D, BM, BN, MODE>& x, f32x16& s, int first_key) {
  // visible iff t0 <= 16 (v / 8) + v % 8 < t1
  const int t0 = x.kvis_lo - first_key - 8 * x.half;
  const int t1 = x.kvis_end - first_key - 8 * x.half;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int o = 16 * (v >> 3) + (v & 7);
    s[v] = ((!x.LEFT || o >= t0) && o < t1) ? s[v] : -INFINITY;
  }
}

__device__ __forceinline__ float max16(const f32x16& s, float m) {
#pragma unroll
  for (int v = 0; v < 16; ++v) m = fmaxf(m, s[v]);
  return m;
}

// P for score i (0 .. 31) of the tile: register i % 16 of accumulator i / 16,
// i.e. PV k-step i / 8, slot i % 8. Scores are exponentiated one at a time so
// the work can be spread evenly between MFMAs, in two stages: exp_issue forms
// p = exp2(s c - m); exp_finish adds it to the row sums and, with the second
// score of a pair, packs the pair to bf16 (and, on masked tiles, splits it
// into hi / lo parts). Issuing the exponentials one MFMA ahead of their use
// hides the latency of the transcendental unit.
template <bool EMU = false>
__device__ __forceinline__ void exp_issue(const f32x16* sc, int i, float c, float nm, float* pe) {
  const float t = __builtin_fmaf(sc[i >> 4][i & 15], c, nm);
  pe[i] = EMU ? exp2_fma(t) : fast_exp2(t);
}

template <bool SPLIT>
__device__ __forceinline__ void exp_finish(int i, float& l_run, float& l_o, const float* pe, uint32_t* ph,
                                           uint32_t* pl) {
  const float p = pe[i];
  l_run += p;
  if (i & 1) {
    const float p0 = pe[i - 1];
    const uint32_t h = pack_bf16x2(p0, p);
    ph[i >> 1] = h;
    if (SPLIT) {
      pl[i >> 1] = pack_bf16x2(p0 - bf16_lo(h), p - bf16_hi(h));
      l_o += p0;
      l_o += p;
    } else {
      l_o = add_bf16x2(h, l_o);
    }
  }
}

template <bool SPLIT>
__device__ __forceinline__ void exp_score(const f32x16* sc, int i, float c, float nm, float& l_run, float& l_o,
                                          float* pe, uint32_t* ph, uint32_t* pl) {
  exp_issue(sc, i, c, nm, pe);
  exp_finish<SPLIT>(i, l_run, l_o, pe, ph, pl);
}

// S^T of one key tile (NA accumulators of 32 keys) for this wave's 32 queries.
template <int D, int BM, int BN, int MODE>
__device__ __forceinline__ void qk_tile(const FwdCtx<D, BM, BN, MODE>& x, const lds_char* Ks,
                                        f32x16 (&s)[FwdCfg<D, BM, BN>::NA]) {
  using T = FwdCfg<D, BM, BN>;
  constexpr int NA = T::NA, PF = T::PF;
  uint4 fr[PF + 1][NA];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
#pragma unroll
    for (int a = 0; a < NA; ++a) fr[kk][a] = lds_ld16(Ks + 32 * a * T::ROW + x.off.row(kk));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < T::KK; ++kk) {
    if (kk + PF < T::KK) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
        fr[(kk + PF) % (PF + 1)][a] = lds_ld16(Ks + 32 * a * T::ROW + x.off.row(kk + PF));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < NA; ++a) s[a] = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][a]), x.qf[kk], kk ? s[a] : zero16());
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pipeline step: tile n's softmax and PV product, tile n + 1's scores.
//  PAR   buffer parity of n;
//  MC    tile n is masked (its scores in sc already hold -inf where invisible);
//  NX    1: tile n + 1 exists and is unmasked; -1: tile n + 1, if there is
//        one, is masked (tiles treated as masked may well be full); -2: tile
//        n + 1 exists and is masked.
// On entry sc holds S(n) and mx this lane's max over it; on return sn holds
// S(n + 1) and mx its max (when tile n + 1 exists).
template <int D, int BM, int BN, int MODE, int PAR, bool MC, int NX>
__device__ __forceinline__ void fwd_step(const FwdCtx<D, BM, BN, MODE>& x, int n, const f32x16 (&sc)[FwdCfg<D, BM, BN>::NA],
                                         f32x16 (&sn)[FwdCfg<D, BM, BN>::NA], f32x16 (&o)[FwdCfg<D, BM, BN>::DB],
                                         float& m_ref, float& l_run, float& l_o, float& mx) {
  using T = FwdCfg<D, BM, BN>;
  constexpr int KK = T::KK, PF = T::PF, DB = T::DB, NA = T::NA, NS = T::NS, NJ = T::NJ;
  constexpr int par = PAR;
  const bool next = NX > 0 || NX == -2 || n + 1 < x.ntiles;

  // every wave is done with tile n - 1; V(n) and K(n + 1) have landed
  wait_vmcnt<0>();
  lds_barrier();
  if (next) {
    if (n + 2 < x.ntiles) issue_tile(x, x.lds0 + par * T::TILE, x.rk, (n + 2) * T::BN);
    issue_tile(x, x.lds0 + T::VBASE + (par ^ 1) * T::TILE, x.rv, (n + 1) * T::BN);
  }
  const lds_char* Kn = x.lds + (par ^ 1) * T::TILE;         // K(n + 1)
  const lds_char* Vc = x.lds + T::VBASE + par * T::TILE;    // V(n)

  uint4 fr[PF + 1][NA];
  if (next) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
#pragma unroll
      for (int a = 0; a < NA; ++a) fr[kk][a] = lds_ld16(Kn + 32 * a * T::ROW + x.off.row(kk));
    }
  }

  // running max: move the reference (and rescale O) only when the tile's max
  // exceeds it by more than the slack, for any lane of the wave
  {
    const float mt = max_xor32(mx);
    const float cand = (mt == -INFINITY) ? -INFINITY : mt * x.c;
    if (__ballot(cand > m_ref + kRescaleSlack)) {
      const float mn = fmaxf(m_ref, cand);
      // 0 when m_ref = -inf (O and l are still 0); rows that have seen no
      // visible key yet keep mn = -inf and must not form exp2(-inf - -inf)
      const float alpha = fast_exp2(m_ref - (mn == -INFINITY ? 0.f : mn));
      m_ref = mn;
      l_run *= alpha;
      l_o *= alpha;
      o_fence<D>(o);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      }
      o_fence<D>(o);
    }
  }
  const float nm = (m_ref == -INFINITY) ? 0.f : -m_ref;

  // The matrix core runs one MFMA at a time and a wave issues in order, so the
  // VALU work is spread in small shares between consecutive MFMAs: each share
  // issues while the MFMA before it executes.
  //
  // phase B: S(n + 1) on the matrix cores (NA KK MFMAs); on the VALU, P(n)
  // scores 0 .. SB - 1 (unmasked tile) or 0 .. 7 (masked tile: its hi / lo
  // parts are formed one PV k-step ahead in phase C instead, which keeps fewer
  // registers live). The last share of phase B holds no score of PV k-step 0.
  constexpr int SB = MC ? 8 : NS * 9 / 16;
  constexpr int NB = NA * KK;
  static_assert(MC || SB * (NB - 1) / NB >= 8, "phase B's last share must not hold k-step 0");
  float pe[NS];
  uint32_t ph[NS / 2], pl[NS / 2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int kk = m / NA, a = m % NA;
    if (next) {
      if (a == 0 && kk + PF < KK) {
#pragma unroll
        for (int b = 0; b < NA; ++b)
          fr[(kk + PF) % (PF + 1)][b] = lds_ld16(Kn + 32 * b * T::ROW + x.off.row(kk + PF));
      }
      sn[a] = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][a]), x.qf[kk], kk ? sn[a] : zero16());
    }
    if (MC) {
#pragma unroll
      for (int i = SB * m / NB; i < SB * (m + 1) / NB; ++i) exp_score<MC>(sc, i, x.c, nm, l_run, l_o, pe, ph, pl);
    } else {
      // this share's exponentials, and the sums / packing of the previous share's
#pragma unroll
      for (int i = SB * m / NB; i < SB * (m + 1) / NB; ++i) {
        if (exp2_emulated(i)) exp_issue<true>(sc, i, x.c, nm, pe);
        else exp_issue(sc, i, x.c, nm, pe);
      }
      if (m > 0) {
#pragma unroll
        for (int i = SB * (m - 1) / NB; i < SB * m / NB; ++i) exp_finish<MC>(i, l_run, l_o, pe, ph, pl);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // phase C: O^T += V(n)^T P(n)^T on the matrix cores, one MFMA unit (PV
  // k-step j, head-dim block db) at a time with the V^T operands read RV - 1
  // units ahead. On the VALU, unmasked tile: the first UC units finish P(n)
  // (scores SB .. NS - 1, each share finished one unit later, the first unit
  // finishing phase B's last share), all of it before the first unit of k-step
  // NJ / 2; the units of the second half of the k-steps take the max of
  // S(n + 1). A masked tile instead forms the next k-step's P during each k-step.
  constexpr int NU = NJ * DB, RV = 3;
  constexpr int UH = (NJ / 2) * DB;  // first unit of the second half
  constexpr int UC = UH - 1;         // units that issue P(n) shares
  static_assert(MC || SB >= 8 * (NJ / 2), "phase C's shares must belong to the second half of the k-steps");
  bf16x8 va[RV];
#pragma unroll
  for (int u = 0; u < RV - 1; ++u) va[u] = tr_operand<D>(Vc + 16 * (u / DB) * T::ROW, x.off, u % DB);
  float mxa = -INFINITY;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = u / DB, db = u % DB;
    if (u + RV - 1 < NU) {
      const int w = u + RV - 1;
      va[w % RV] = tr_operand<D>(Vc + 16 * (w / DB) * T::ROW, x.off, w % DB);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 pb = as_bf16x8(make_uint4(ph[4 * j], ph[4 * j + 1], ph[4 * j + 2], ph[4 * j + 3]));
    pv_mfma<D>(o[db], va[u % RV], pb);
    if (MC) {
      const bf16x8 pq = as_bf16x8(make_uint4(pl[4 * j], pl[4 * j + 1], pl[4 * j + 2], pl[4 * j + 3]));
      pv_mfma<D>(o[db], va[u % RV], pq);
      if (j + 1 < NJ) {
#pragma unroll
        for (int i = 8 * (j + 1) + 8 * db / DB; i < 8 * (j + 1) + 8 * (db + 1) / DB; ++i)
          exp_score<MC>(sc, i, x.c, nm, l_run, l_o, pe, ph, pl);
      }
    } else if (u <= UC) {
      if (u < UC) {
#pragma unroll
        for (int i = SB + (NS - SB) * u / UC; i < SB + (NS - SB) * (u + 1) / UC; ++i) {
          if (exp2_emulated(i)) exp_issue<true>(sc, i, x.c, nm, pe);
          else exp_issue(sc, i, x.c, nm, pe);
        }
      }
      const int f0 = u ? SB + (NS - SB) * (u - 1) / UC : SB * (NB - 1) / NB;
      const int f1 = u ? SB + (NS - SB) * u / UC : SB;
#pragma unroll
      for (int i = f0; i < f1; ++i) exp_finish<MC>(i, l_run, l_o, pe, ph, pl);
    }
    if (next && u >= UH) {
      // mask and max of S(n + 1): NA x 16 values spread over the units of the
      // second half of the k-steps
      const int e = u - UH;
#pragma unroll
      for (int i = 16 * NA * e / (NU - UH); i < 16 * NA * (e + 1) / (NU - UH); ++i) {
        const int v = i & 15;
        if (NX < 0) {
          const int base = (n + 1) * T::BN + 32 * (i >> 4) + 8 * x.half;
          const int o = 16 * (v >> 3) + (v & 7);
          sn[i >> 4][v] = ((!x.LEFT || o >= x.kvis_lo - base) && o < x.kvis_end - base) ? sn[i >> 4][v] : -INFINITY;
        }
        mxa = fmaxf(mxa, sn[i >> 4][v]);
      }
      asm volatile("" : "+v"(mxa));  // keep this unit's share of the max here
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  mx = mxa;  // meaningless when there is no tile n + 1
}

// MODE 0: full attention; 1: the visible keys of a row end at a band edge
// (causal and / or a right window bound); 2: they also start at one (a left
// window bound), so an item may begin with masked tiles.
struct NoHook {
  __device__ void operator()() const {}
};

// The lane index, formed where it is written: a volatile asm statement is not
// hoisted out of a loop, so no register holds the lane index across it.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// SPLIT: the workgroup runs one chunk of the item's key tiles and writes the
// chunk's partial result (FwdParams::part_o / part_l) instead of out / lse.
//
// One work item: logical index L = (query block rank, key chunk) x query head,
// heads innermost, so that the r heads of a KV group are adjacent indices.
// hook() runs exactly once per call, on every path: right after the
// prologue's wait for all of the item's loads (or, for an item without key
// tiles, in place of it). The persistent kernel publishes its next item there,
// from an atomic issued before the call, which by then has completed.
// With a hook, `wave` is this wave's index in the workgroup (wave-uniform) and
// the thread index is formed from it and the lane, so that no thread-index
// register stays live across the persistent kernel's loop.
template <int D, int BM, int BN, int MODE, bool WRITE_LSE, bool SPLIT, class Hook = NoHook>
__device__ __forceinline__ void fwd_item(const FwdParams& p, int64_t L, uint16_t* smem, const Hook& hook = Hook(),
                                         int wave = 0) {
  using T = FwdCfg<D, BM, BN>;
  constexpr int NA = T::NA;

  const int r = p.Hq / p.Hkv;
  const int heads = p.Hq >> p.hw_log2;  // head sets of hw heads
  const int hs = (int)(L % heads);
  int rank, split = 0;
  if (SPLIT) {
    const int64_t unit = L / heads;
    split = (int)(unit % p.splits);
    rank = (int)(unit / p.splits);
  } else {
    rank = (int)(L / heads);
  }
  Item item;
  if (!decode_item<false>(p.cu_q, p.cu_k, p.num_seqs, p.bm, p.levels, rank, item)) {
    hook();
    return;
  }
  const int g = (hs << p.hw_log2) / r;
  const int mblk = item.m, cq = item.cq, Lq = item.Lq, ck = item.ck, Lk = item.Lk;

  FwdCtx<D, BM, BN, MODE> x;
  x.lds = (const lds_char*)smem;
  x.lds0 = lds_addr((lds_char*)smem);
  // In the persistent kernel's loop the thread index is made opaque, so that
  // the lane-derived values below are formed per item instead of being
  // hoisted out of the loop and held in registers through the hot loop.
  int tid;
  if constexpr (std::is_same<Hook, NoHook>::value) {
    tid = threadIdx.x;
  } else {
    tid = wave * 64 + lane_id_here();
  }
  x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  x.half = lane >> 5;
  // this wave's query head and 32-row part of the block
  const int h = (hs << p.hw_log2) + (x.wave & (p.hw - 1));
  const int wrow = (x.wave >> p.hw_log2) * 32;
  // query blocks are aligned toward the end of the sequence: the first block
  // starts `lead` rows before row 0 (the padding of the last block rounded
  // down to whole key tiles), so that a partial block is mostly the first one,
  // which under a causal mask sees the fewest keys, while block starts stay on
  // the key-tile grid (a block's causal diagonal then crosses BM / BN tiles)
  const int q0 = mblk * p.bm - query_lead(Lq, p.bm, T::BN);
  const int qi = q0 + wrow + (lane & 31);  // this lane's query row (sequence-relative)
  const bool qvalid = qi >= 0 && qi < Lq;

  // key tiles of this block, [t_lo, t_hi), and the unmasked ones among them,
  // [f_lo, f_hi): every key below Lk and inside every row's band
  constexpr bool BAND = MODE > 0;
  int t_lo = 0, t_hi = ceil_div(Lk, T::BN), f_lo = 0, f_hi = Lk / T::BN;
  if (BAND) {
    const TileSpan ts = key_tiles(max(q0, 0), min(q0 + p.bm, Lq) - 1, T::BN, Lq, Lk, MODE == 2 ? p.wl : -1, p.wr);
    t_lo = ts.lo;
    t_hi = ts.hi;
    f_lo = ts.full_lo;
    f_hi = ts.full_hi;
  }
  if (SPLIT) {
    // chunk `split` of the item's tiles: ceil(n / splits) tiles each, the last
    // ones possibly empty (then only the -inf row sums are written)
    const int chunk = ceil_div(t_hi - t_lo, p.splits);
    const int s_lo = min(t_hi, t_lo + split * chunk);
    t_hi = min(t_hi, s_lo + chunk);
    t_lo = s_lo;
    if (t_lo >= t_hi) {
      if (qvalid && x.half == 0) {
        const int64_t li = ((int64_t)split * 2 * p.Hq + h) * p.total_q + cq + qi;
        p.part_l[li] = -INFINITY;
        p.part_l[li + (int64_t)p.Hq * p.total_q] = -INFINITY;
      }
      hook();
      return;
    }
  }
  if (MODE == 2 || SPLIT) {  // see below
    t_lo = __builtin_amdgcn_readfirstlane(t_lo);
    t_hi = __builtin_amdgcn_readfirstlane(t_hi);
    f_lo = __builtin_amdgcn_readfirstlane(f_lo);
    f_hi = __builtin_amdgcn_readfirstlane(f_hi);
  }
  x.ntiles = t_hi;
  x.kvis_lo = (MODE == 2) ? band_lo(qi, Lq, Lk, p.wl) : 0;
  x.kvis_end = BAND ? band_hi(qi, Lq, Lk, p.wr) : Lk;
  // tile order (local indices): the unmasked tiles [0, nm), then the masked
  // ones. With a left window bound (MODE 2) the first tiles cross some row's
  // left band edge: the nh (even) of them that lie left of every row's right
  // edge are masked by the step before them and then take the unmasked P path,
  // when the window is at least a tile wide (every row that reaches such a tile
  // then sees at least BN keys, as in the unmasked tiles of any item). Narrower
  // windows run every tile as a masked step.
  const int ntot = t_hi - t_lo;
  int nh = 0;
  int nm = SPLIT ? max(0, min(f_hi, t_hi) - t_lo) : f_hi;
  if (MODE == 2) left_edge_tiles(t_lo, t_hi, f_lo, f_hi, p.wl, T::BN, nh, nm);
  // The tile counts are the same in every lane; saying so keeps the loops'
  // control in scalar registers where the compiler does not prove it (with a
  // left band edge or split-KV chunks; vector loop bounds there cost registers
  // the pipeline needs, and the kernels spilled).
  if (MODE == 2 || SPLIT) {
    nm = __builtin_amdgcn_readfirstlane(nm);
    nh = __builtin_amdgcn_readfirstlane(nh);
  }
  x.c = p.scale_log2;

  // K / V buffer resources for this (sequence, KV head): rows past Lk read as 0
  const uint32_t pitch = (uint32_t)p.Hkv * D * 2;
  x.tile_bytes = pitch * T::BN;
  const int64_t kvoff = ((int64_t)ck * p.Hkv + g) * D;
  x.rk = head_rows_rsrc<D>(p.k + kvoff, Lk, pitch);
  x.rv = head_rows_rsrc<D>(p.v + kvoff, Lk, pitch);
  if constexpr (FwdCtx<D, BM, BN, MODE>::ONE_VOFF) {
    static_assert(T::WAVES % 4 == 0 && (T::KV::ROWS_PER_DMA * T::WAVES) % 16 == 0,
                  "the rows of a wave's copies must share one chunk swizzle");
    const int row = x.wave * T::KV::ROWS_PER_DMA + lane / T::KV::CPR;
    x.voff[0] = (uint32_t)row * pitch + (uint32_t)(((lane % T::KV::CPR) ^ swz<D>(row)) * 16);
    x.round_bytes = (uint32_t)(T::KV::ROWS_PER_DMA * T::WAVES) * pitch;
  } else {
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
      const int row = (x.wave * T::DMA + i) * T::KV::ROWS_PER_DMA + lane / T::KV::CPR;
      const int cidx = (lane % T::KV::CPR) ^ swz<D>(row);
      x.voff[i] = (uint32_t)row * pitch + (uint32_t)cidx * 16u;
    }
  }

  // prologue copies: K(t_lo) -> K0, V(t_lo) -> V0, K(t_lo + 1) -> K1; then Q^T
  // into VGPRs. Buffer parity follows the local tile index n - t_lo.
  if (ntot > 0) {
    issue_tile(x, x.lds0, x.rk, t_lo * T::BN);
    issue_tile(x, x.lds0 + T::VBASE, x.rv, t_lo * T::BN);
    if (ntot > 1) issue_tile(x, x.lds0 + T::TILE, x.rk, (t_lo + 1) * T::BN);
  }
  {
    // Q^T operand: 8 consecutive head-dims of this lane's query per k-step
    // (sign-flipped when the scale is negative, so the scale applied is positive)
    const uint16_t* qrow = p.q + ((int64_t)(cq + (qvalid ? qi : 0)) * p.Hq + h) * D + 8 * x.half;
    const uint32_t flip = p.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      uint4 u = qvalid ? ld16(qrow + 16 * kk) : zero_u4();
      u.x ^= flip;
      u.y ^= flip;
      u.z ^= flip;
      u.w ^= flip;
      x.qf[kk] = as_bf16x8(u);
    }
  }
  operand_offsets<D>(x.off, lane);

  f32x16 o[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) o[db] = zero16();
  float m_ref = -INFINITY;
  float l_run = 0.f;  // sum of P (fp32): the LSE
  float l_o = 0.f;    // sum of the P values as they enter the PV product: normalises O
  float mx = -INFINITY;
  f32x16 sa[NA], sb[NA];

  if (ntot > 0) {
    wait_vmcnt<0>();
    hook();
    lds_barrier();
    qk_tile(x, x.lds, sa);
    if (MODE == 2 || nm <= 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a) mask_scores(x, sa[a], t_lo * T::BN + 32 * a);
    }
#pragma unroll
    for (int a = 0; a < NA; ++a) mx = max16(sa[a], mx);
  } else {
    hook();
  }

  // S(n) lives in sa for even local index t = n - t_lo, sb for odd t; steps
  // get the absolute tile index n. (t_lo is 0 unless MODE 2 or SPLIT.)
  int t = 0;
  if (nm > 0) {
    if (MODE == 2) {
      // left-edge tiles: each step masks the next tile's scores
      // (nh < nm <= ntot: a next tile always exists here)
      for (; t < nh; t += 2) {
        fwd_step<D, BM, BN, MODE, 0, false, -2>(x, t_lo + t, sa, sb, o, m_ref, l_run, l_o, mx);
        fwd_step<D, BM, BN, MODE, 1, false, -2>(x, t_lo + t + 1, sb, sa, o, m_ref, l_run, l_o, mx);
      }
    }
    // steady state, unrolled by two so the buffer parity is a constant: tiles
    // t and t + 1 both unmasked
    for (; t + 3 <= nm; t += 2) {
      fwd_step<D, BM, BN, MODE, 0, false, 1>(x, t_lo + t, sa, sb, o, m_ref, l_run, l_o, mx);
      fwd_step<D, BM, BN, MODE, 1, false, 1>(x, t_lo + t + 1, sb, sa, o, m_ref, l_run, l_o, mx);
    }
    // last unmasked step (t is even); the tiles after it are all treated as
    // masked, which is exact for full tiles too
    fwd_step<D, BM, BN, MODE, 0, false, -1>(x, t_lo + t, sa, sb, o, m_ref, l_run, l_o, mx);
    ++t;
  } else if (ntot > 0) {
    fwd_step<D, BM, BN, MODE, 0, true, -1>(x, t_lo, sa, sb, o, m_ref, l_run, l_o, mx);
    t = 1;
  }
  // masked tail from an odd t, unrolled by two like the steady state
  while (t < ntot) {
    fwd_step<D, BM, BN, MODE, 1, true, -1>(x, t_lo + t, sb, sa, o, m_ref, l_run, l_o, mx);
    if (++t >= ntot) break;
    fwd_step<D, BM, BN, MODE, 0, true, -1>(x, t_lo + t, sa, sb, o, m_ref, l_run, l_o, mx);
    ++t;
  }

  // epilogue: O = O / l, LSE = ln(2) * (m + log2 l)
  o_fence<D>(o);
  const float l_tot = add_xor32(l_run);
  const float lo_tot = add_xor32(l_o);
  if (SPLIT) {
    if (qvalid) {
      const float inv = (lo_tot > 0.f) ? 1.f / lo_tot : 0.f;
      float* orow = p.part_o + (((int64_t)split * p.total_q + cq + qi) * p.Hq + h) * D + 4 * x.half;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) store_acc_row_f32(orow + db * 32, o[db], inv);
      if (x.half == 0) {
        const bool any = l_tot > 0.f && m_ref != -INFINITY;
        const int64_t li = ((int64_t)split * 2 * p.Hq + h) * p.total_q + cq + qi;
        p.part_l[li] = any ? m_ref + log2f(l_tot) : -INFINITY;
        p.part_l[li + (int64_t)p.Hq * p.total_q] = (any && lo_tot > 0.f) ? m_ref + log2f(lo_tot) : -INFINITY;
      }
    }
    return;
  }
  if (qvalid) {
    const float inv = (lo_tot > 0.f) ? 1.f / lo_tot : 0.f;
    uint16_t* orow = p.out + ((int64_t)(cq + qi) * p.Hq + h) * D + 4 * x.half;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) store_acc_row(orow + db * 32, o[db], inv);
    if (WRITE_LSE && x.half == 0) {
      p.lse[(int64_t)h * p.total_q + cq + qi] =
          (l_tot > 0.f && m_ref != -INFINITY) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// One workgroup per work item; the block index is spread over the XCDs so that
// the r heads of a KV group (adjacent logical indices) run on one XCD and share
// K / V in its L2.
template <int D, int BM, int BN, int MODE, bool WRITE_LSE, bool SPLIT = false>
__global__ __launch_bounds__((FwdCfg<D, BM, BN>::NT), (FwdCfg<D, BM, BN>::MIN_BLOCKS_PER_CU)) void fwd_kernel(
    FwdParams p) {
  extern __shared__ __align__(16) uint16_t smem[];
  fwd_item<D, BM, BN, MODE, WRITE_LSE, SPLIT>(p, xcd_logical(blockIdx.x, (p.Hq / p.Hkv) >> p.hw_log2), smem);
}

// Persistent scheduling (FlashAttention repository guide, Core Abstractions:
// the varlen-aware persistent tile scheduler): as many workgroups as the chip
// holds at once, each running work items until none is left. The n_items
// logical indices (longest first, a multiple of 8 r) are dealt to 8 queues by
// KV group: queue q holds the groups q, q + 8, q + 16, ... in order. A
// workgroup takes items from the queue of the XCD it runs on, then from the
// other queues in turn. The heads of a group thus mostly share one XCD's L2,
// and XCDs that run faster (under the board power limit they do not all hold
// the same clock) take more of the work, which a fixed block-to-XCD assignment
// cannot do. Every workgroup leaves the loop once all queues are exhausted;
// the last one to finish returns the counters to 0 for the next call.
// The kernel's FwdParams argument, in the kernel-argument segment (its first bytes).
typedef const __attribute__((address_space(4))) FwdParams* KernargParams;

template <int D, int BM, int BN, int MODE, bool WRITE_LSE>
__global__ __launch_bounds__((FwdCfg<D, BM, BN>::NT), (FwdCfg<D, BM, BN>::MIN_BLOCKS_PER_CU)) void
fwd_kernel_persistent(FwdParams p, unsigned int n_items) {
  using T = FwdCfg<D, BM, BN>;
  extern __shared__ __align__(16) uint16_t smem[];
  // LDS after the K / V buffers: the current and the next item (alternating),
  // then thread 0's count of queues found empty so far
  // (plain LDS accesses: the barriers order them)
  int* slot = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + T::LDS_BYTES);
  const unsigned int r = (unsigned int)((p.Hq / p.Hkv) >> p.hw_log2);  // items per KV group and block
  const unsigned int per_queue = n_items / kNumXcd;  // items per queue (whole groups)
  // thread 0, tested without keeping the thread index live across the loop
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto first = [&]() { return wave == 0 && lane_id_here() == 0; };
  unsigned int xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
  // Thread 0: the item behind ticket idx of queue (xcc + k) % 8, else the next
  // queues in turn (a ticket past the end of a queue is discarded); -1 once
  // every queue is empty. Returns the queues found empty in k.
  // (Only lane 0 of wave 0 runs it: readfirstlane keeps the division scalar.)
  auto resolve = [&](unsigned int idx, unsigned int& k) -> int {
    while (k < (unsigned int)kNumXcd) {
      const unsigned int q = (xcc + k) % kNumXcd;
      const unsigned int i = __builtin_amdgcn_readfirstlane(idx);
      if (i < per_queue) return (int)(((i / r) * kNumXcd + q) * r + i % r);
      if (++k < (unsigned int)kNumXcd) idx = atomicAdd(p.sched + (xcc + k) % kNumXcd, 1u);
    }
    return -1;
  };
  if (first()) {
    unsigned int k = 0;
    slot[0] = resolve(atomicAdd(p.sched + xcc % kNumXcd, 1u), k);
    slot[2] = (int)k;
  }
  __syncthreads();
  for (int cur = 0;; cur ^= 1) {
    const int L = __builtin_amdgcn_readfirstlane(slot[cur]);  // the same in every lane
    if (L < 0) break;
    // claim the next item now; fwd_item's first wait completes the atomic, and
    // the hook publishes the item for the loop's next turn
    unsigned int ticket = 0;
    if (first() && slot[2] < kNumXcd) ticket = atomicAdd(p.sched + (xcc + slot[2]) % kNumXcd, 1u);
    auto publish = [&]() {
      if (first()) {
        unsigned int k = (unsigned int)slot[2];
        slot[cur ^ 1] = resolve(ticket, k);
        slot[2] = (int)k;
      }
    };
    // The item reads the parameters through a pointer the compiler cannot see
    // through, so that it loads them inside the item, as the one-item kernel
    // does, instead of holding all of them in scalar registers across the loop
    // (which spills the hot loop).
    KernargParams pi = (KernargParams)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pi));
    fwd_item<D, BM, BN, MODE, WRITE_LSE, false>(*(const FwdParams*)pi, L, smem, publish, wave);
    __syncthreads();  // the next item is published; every wave is done with this item's LDS
  }
  if (first()) {
    __threadfence();
    if (atomicAdd(p.sched + kNumXcd, 1u) == gridDim.x - 1) {
      for (int q = 0; q <= kNumXcd; ++q) atomicExch(p.sched + q, 0u);
    }
  }
}

// Kernel parameters of a validated call (the grid's query blocks have bm rows).
inline FwdParams fwd_params(const FwdArgs& a, int bm) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.out = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.num_seqs = a.num_seqs;
  p.total_q = (int)a.total_q;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  static_assert(FwdCfg<128, kQueryBlock, 64>::WAVES == 4, "block_heads assumes four waves");
  p.hw = (bm == kQueryBlock) ? block_heads(a.Hq / a.Hkv) : 1;
  p.hw_log2 = log2_small(p.hw);
  p.bm = bm / p.hw;
  p.levels = ceil_div(a.max_q, p.bm);
  // a zero (or tiny) scale becomes the smallest normal float: the scores then
  // all map to exp2(~0) = 1 as for scale 0, while masked scores (-inf) stay -inf
  p.scale_log2 = fmaxf(fabsf(a.scale) * kLog2e, FLT_MIN);
  p.neg_scale = a.scale < 0.f ? 1 : 0;
  const Band bd = band_of(a);
  p.wl = bd.wl;
  p.wr = bd.wr;
  p.part_o = nullptr;
  p.part_l = nullptr;
  p.splits = 1;
  p.sched = nullptr;
  return p;
}

}  // namespace av

#endif  // AV_FWD_KERNEL_H
