// av_bwd_d256.hip — backward main kernels for head dim 256: the dK / dV and dQ
// products of the FlashAttention repository guide's backward (Backward
// Kernels), after the preprocess kernel of av_bwd.hip (Delta, lse2).
//
// At head_dim 256 a wave's accumulators alone take 256 (dK + dV for 32 keys) or
// 128 (dQ for 32 queries) registers per lane, so both kernels run one wave per
// SIMD with the accumulators pinned to AGPRs (inline-asm MFMA: left to itself
// the register allocator moves loop-carried accumulators between register
// files). The asm is opaque to the compiler's hazard checks, so it carries its
// own padding: s_nop 1 before each MFMA covers a VALU-written operand, and
// acc_fence() separates MFMA writes of the accumulators from their VALU reads.
//
//  bwd_dkdv256_kernel  key-stationary: a workgroup owns 128 keys (32 per wave)
//                      of one KV head and one split of that head's query
//                      heads, and loops over every 32-row query block that can
//                      see the keys: S = Q K^T, P = exp2(S scale log2 e - lse2),
//                      dP = dO V^T, dS = P (dP - Delta), dV += P^T dO,
//                      dK += dS^T Q. K^T stays in VGPRs, the item's V block is
//                      copied to LDS once (64 KB; registers cannot hold it next
//                      to the 256 accumulator registers); Q / dO tiles and the
//                      rows' lse2 / Delta arrive by buffer-load DMA,
//                      double-buffered. With one split the group sum is done in
//                      registers and dK / dV are written directly; with more
//                      (few key blocks per KV head, so too few work items to
//                      fill the chip or to balance causal work), each split
//                      writes fp32 partial sums that bwd_dkdv_reduce_kernel adds
//                      in split order: deterministic, no atomics.
//  bwd_dq256_kernel    query-stationary: a workgroup owns 128 query rows (32 per
//                      wave) of one head and loops over the visible 32-key tiles
//                      in ascending order: dQ += dS K. 32-key tiles keep the two
//                      double-buffered K / V stages within 64 KB, so every LDS
//                      operand address is a register plus an immediate.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "av_bwd.h"
#include "av_common.h"
#include "av_launch.h"
#include "av_tiles.h"

namespace av {

hipError_t launch_dkdv_reduce(const float* part_dk, const float* part_dv, uint16_t* dk, uint16_t* dv, int64_t n8,
                              int splits, float scale, hipStream_t stream);

namespace {

constexpr int kD = 256;
constexpr int kKK = kD / 16;  // k-steps of a contraction over head_dim
constexpr int kDB = kD / 32;  // 32-wide head-dim blocks of an accumulator

// acc += A B with the accumulator in AGPRs (see the file comment).
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc (+)= A B with the accumulator pinned to VGPRs (the S / dP products, which
// the VALU reads next); the first k-step starts from zero. vgpr_fence() gives
// an MFMA result the wait states it needs before the VALU reads it.
__device__ __forceinline__ void mfma_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// Operand registers loaded from memory before a tile loop are consumed here, so
// that the compiler waits for those loads once, before the loop. Left pending
// into the loop, its wait at their first use there would also wait for the
// tile copies issued just before it (the copies count in the same counter),
// in every iteration.
__device__ __forceinline__ void settle(bf16x8 (&r)[kKK]) {
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) asm volatile("" : "+v"(r[kk]));
}
__device__ __forceinline__ void vgpr_fence(f32x16& a, f32x16& b) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// 24 wait states, with the accumulators as operands so that no read or write
// of them moves across: more than an MFMA result needs before a VALU read.
__device__ __forceinline__ void acc_fence(f32x16 (&a)[kDB]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]));
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------

struct Dkdv256 {
  static constexpr int NT = 256;
  static constexpr int BNK = 128;  // keys per workgroup (32 per wave)
  static constexpr int BMQ = 32;   // query rows per step
  static_assert(BNK == kKeyBlock && BMQ == query_step(kD), "tile shapes of the host-side plan");
  using QT = RowTile<kD, BMQ>;
  static constexpr int ROW = QT::ROW;
  static constexpr int TILE = QT::BYTES;     // 16 KB
  static constexpr int STAGE = 2 * TILE;     // Q tile, then dO tile
  using VT = RowTile<kD, BNK>;
  static constexpr int VBASE = 2 * STAGE;               // the item's V block (64 KB)
  static constexpr int F32 = VBASE + VT::BYTES;         // lse2 / Delta of both stages
  static constexpr int F32_STAGE = 512;                 // lse2[64] then Delta[64] (a copy moves 64 rows)
  static constexpr size_t LDS_BYTES = F32 + 2 * F32_STAGE;
  static constexpr int VDMA_PER_WAVE = VT::DMAS / 4;
  static constexpr int DMA_PER_WAVE = 2 * QT::DMAS / 4;  // Q and dO copies
  static constexpr int PF = 1;                           // operand prefetch distance (k-steps)
  static constexpr int RV = 2;                           // ring of transposed operands
  static_assert(2 * STAGE <= 65536, "tile offsets must fit the 16-bit LDS immediate");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void issue_qdo256(uint32_t lds0, int stage, const i32x4& rq, const i32x4& rdo,
                                             const i32x4& rl, const i32x4& rd, uint32_t pitch, int m0, int wave,
                                             int lane) {
  using T = Dkdv256;
  const uint32_t st = lds0 + stage * T::STAGE;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;
    const bool is_do = qd >= T::QT::DMAS;
    tile_dma<kD, T::BMQ>(st + (is_do ? T::TILE : 0), is_do ? rdo : rq, pitch, m0, is_do ? qd - T::QT::DMAS : qd,
                         lane);
  }
  const uint32_t f = lds0 + T::F32 + stage * T::F32_STAGE;
  if (wave == 0) rows64_f32_dma(f, rl, m0, lane);
  if (wave == 1) rows64_f32_dma(f + 256, rd, m0, lane);
}

// One step: the 32 query rows at sequence row m0 against this wave's 32 keys.
// B operand of dP = dO V^T for k-step kk: lane l holds head-dims 16 kk +
// 8 (l / 32) .. + 7 of key row (wave's key l % 32) of the V block in LDS;
// vrow[] holds the byte addresses of the first 16 chunks of that row (chunk
// c + 16 lies 256 bytes after chunk c).
__device__ __forceinline__ uint4 v_operand(const lds_char* lds, const uint32_t* vrow, int kk) {
  return lds_ld16(lds + vrow[kk % 8] + 256 * (kk / 8));
}

template <bool MASK, bool LEFT>
__device__ __forceinline__ void dkdv256_step(const lds_char* lds, const lds_char* Qs, const lds_char* dOs,
                                             const float* lse2_s, const float* dlt_s, const bf16x8* kf,
                                             const uint32_t* vrow, f32x16 (&dk)[kDB], f32x16 (&dv)[kDB], float c,
                                             int rlo, int rhi, const OperandOffsets<kD>& off, int half) {
  using T = Dkdv256;
  constexpr int PF = T::PF, RV = T::RV;
  // S (query rows x keys) and dP: two independent chains, LDS operands
  // (Q and dO rows, V rows) fetched PF k-steps ahead
  f32x16 s, dp;
  uint4 fr[PF + 1][3];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    fr[kk][0] = lds_ld16(Qs + off.row(kk));
    fr[kk][1] = lds_ld16(dOs + off.row(kk));
    fr[kk][2] = v_operand(lds, vrow, kk);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    if (kk + PF < kKK) {
      fr[(kk + PF) % (PF + 1)][0] = lds_ld16(Qs + off.row(kk + PF));
      fr[(kk + PF) % (PF + 1)][1] = lds_ld16(dOs + off.row(kk + PF));
      fr[(kk + PF) % (PF + 1)][2] = v_operand(lds, vrow, kk + PF);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kk == 0) {
      mfma_vgpr0(s, as_bf16x8(fr[0][0]), kf[0]);
      mfma_vgpr0(dp, as_bf16x8(fr[0][1]), as_bf16x8(fr[0][2]));
    } else {
      mfma_vgpr(s, as_bf16x8(fr[kk % (PF + 1)][0]), kf[kk]);
      mfma_vgpr(dp, as_bf16x8(fr[kk % (PF + 1)][1]), as_bf16x8(fr[kk % (PF + 1)][2]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  vgpr_fence(s, dp);
  // dV += P^T dO and dK += dS^T Q, one (k-step ks of 16 queries, head-dim
  // block db) unit at a time; the transposed dO / Q operands are read RV - 1
  // units ahead.
  bf16x8 tdo[RV], tq[RV];
#pragma unroll
  for (int u = 0; u < RV - 1; ++u) {
    tdo[u] = tr_operand<kD>(dOs + 16 * (u / kDB) * T::ROW, off, u % kDB);
    tq[u] = tr_operand<kD>(Qs + 16 * (u / kDB) * T::ROW, off, u % kDB);
  }
  // P and dS of k-step ks (8 queries per lane: 16 ks + 8 half + e). k-step 0
  // is formed before the first unit; k-step 1 is spread over the units of
  // k-step 0 (one score issued per unit, finished one unit later), so that its
  // vector work issues between those MFMAs instead of as one block.
  float l2[2][8], dl[2][8];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int qo = 16 * ks + 8 * half;
    const float4 a0 = *reinterpret_cast<const float4*>(lse2_s + qo);
    const float4 a1 = *reinterpret_cast<const float4*>(lse2_s + qo + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(dlt_s + qo);
    const float4 b1 = *reinterpret_cast<const float4*>(dlt_s + qo + 4);
    l2[ks][0] = a0.x; l2[ks][1] = a0.y; l2[ks][2] = a0.z; l2[ks][3] = a0.w;
    l2[ks][4] = a1.x; l2[ks][5] = a1.y; l2[ks][6] = a1.z; l2[ks][7] = a1.w;
    dl[ks][0] = b0.x; dl[ks][1] = b0.y; dl[ks][2] = b0.z; dl[ks][3] = b0.w;
    dl[ks][4] = b1.x; dl[ks][5] = b1.y; dl[ks][6] = b1.z; dl[ks][7] = b1.w;
  }
  float pe[8], pm[8], dsv[8];
  uint32_t pw[2][4], sw[2][4];
  auto issue = [&](int ks, int e) { pe[e] = fast_exp2(__builtin_fmaf(s[8 * ks + e], c, -l2[ks][e])); };
  auto finish = [&](int ks, int e) {
    float pv = pe[e];
    if (MASK) {
      const int row = 16 * ks + 8 * half + e;
      pv = (row >= rlo && (!LEFT || row <= rhi)) ? pv : 0.f;
    }
    pm[e] = pv;
    dsv[e] = pv * (dp[8 * ks + e] - dl[ks][e]);
    if (e & 1) {
      pw[ks][e >> 1] = pack_bf16x2(pm[e - 1], pm[e]);
      sw[ks][e >> 1] = pack_bf16x2(dsv[e - 1], dsv[e]);
    }
  };
#pragma unroll
  for (int e = 0; e < 8; ++e) issue(0, e);
#pragma unroll
  for (int e = 0; e < 8; ++e) finish(0, e);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < 2 * kDB; ++u) {
    const int ks = u / kDB, db = u % kDB;
    if (u + RV - 1 < 2 * kDB) {
      const int w = u + RV - 1;
      tdo[w % RV] = tr_operand<kD>(dOs + 16 * (w / kDB) * T::ROW, off, w % kDB);
      tq[w % RV] = tr_operand<kD>(Qs + 16 * (w / kDB) * T::ROW, off, w % kDB);
    }
    // k-step 1's scores: issue score u, finish score u - 1 (the last one just
    // before k-step 1's first unit)
    if (u < 8) issue(1, u);
    if (u >= 1 && u <= 8) finish(1, u - 1);
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 pb = as_bf16x8(make_uint4(pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]));
    const bf16x8 sb = as_bf16x8(make_uint4(sw[ks][0], sw[ks][1], sw[ks][2], sw[ks][3]));
    mfma_agpr(dv[db], tdo[u % RV], pb);
    mfma_agpr(dk[db], tq[u % RV], sb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// BAND: the visible keys of a row form a band (causal and / or a local window).
// LEFT: the band has a left bound (window_left >= 0); without one, masked steps
// test only a key's first visible row.
template <bool BAND, bool LEFT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv256_kernel(BwdParams p) {
  using T = Dkdv256;
  extern __shared__ __align__(16) uint16_t smem[];
  lds_char* lds = (lds_char*)smem;

  // work item: (sequence, key block) ranked by descending work, x KV heads x
  // query-head splits. The rank's level counts key blocks from the end of the
  // sequence, so the blocks seen by the most query rows come first. Items are
  // taken in block order, which the dispatcher deals to the 8 XCDs round-robin:
  // with 8 splits (or a divisor of 8) an XCD then runs one split, i.e. one set
  // of query heads, for many key blocks at once, and those stream the same Q /
  // dO rows through its L2. (Keeping a key block's splits on one XCD instead
  // shares only the small K / V block: 2x16K non-causal then fetched 9.5 GB per
  // launch against 2.5 GB this way, and the backward ran 3-7% slower.)
  const int S = p.splits;
  const int64_t L = blockIdx.x;
  const int rank = (int)(L / ((int64_t)p.Hkv * S));
  const int rem = (int)(L % ((int64_t)p.Hkv * S));
  const int g = rem / S;
  const int split = rem % S;
  Item item;
  if (!decode_item<true>(p.cu_q, p.cu_k, p.num_seqs, T::BNK, p.levels, rank, item)) return;
  const int lvl = item.m, cq = item.cq, Lq = item.Lq, ck = item.ck, Lk = item.Lk;
  const int n0 = (ceil_div(Lk, T::BNK) - 1 - lvl) * T::BNK;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int kj = n0 + wave * 32 + col;  // this lane's key (sequence-relative)
  const bool kvalid = kj < Lk;
  const int r = p.Hq / p.Hkv;
  const int hper = r / S;  // query heads of this split: g r + split hper + [0, hper)

  // query steps [sfirst, sfirst + nsteps) whose rows see a key of this block,
  // and among them the unmasked ones [s_full_lo, s_full_hi) (relative)
  int sfirst = 0, nsteps = ceil_div(Lq, T::BMQ), s_full_lo = 0, s_full_hi = nsteps;
  if (BAND) {
    const TileSpan ts = query_steps(n0, min(n0 + T::BNK, Lk) - 1, T::BMQ, Lq, Lk, p.wl, p.wr);
    sfirst = ts.lo;
    nsteps = ts.hi - ts.lo;
    s_full_lo = ts.full_lo - sfirst;
    s_full_hi = ts.full_hi - sfirst;
  }
  const int total = (nsteps > 0) ? nsteps * hper : 0;

  const uint32_t pitch = (uint32_t)p.Hq * kD * 2;
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int it, int stage) {
    const int h = g * r + split * hper + it / nsteps;
    const int m0 = (sfirst + it % nsteps) * T::BMQ;
    const int64_t qoff = ((int64_t)cq * p.Hq + h) * kD;
    const i32x4 rq = head_rows_rsrc<kD>(p.q + qoff, Lq, pitch);
    const i32x4 rdo = head_rows_rsrc<kD>(p.dout + qoff, Lq, pitch);
    const int64_t roff = (int64_t)h * p.total_q + cq;
    const i32x4 rl = make_rsrc(p.lse2 + roff, (uint32_t)Lq * 4u);
    const i32x4 rd = make_rsrc(p.delta + roff, (uint32_t)Lq * 4u);
    issue_qdo256(lds0, stage, rq, rdo, rl, rd, pitch, m0, wave, lane);
  };
  if (total > 0) {
    // the item's V block (rows n0 .. n0 + 127; rows past Lk read as 0), once
    const uint32_t kvpitch = (uint32_t)p.Hkv * kD * 2;
    const i32x4 rv = head_rows_rsrc<kD>(p.v + ((int64_t)ck * p.Hkv + g) * kD, Lk, kvpitch);
#pragma unroll
    for (int i = 0; i < T::VDMA_PER_WAVE; ++i)
      tile_dma<kD, T::BNK>(lds0 + T::VBASE, rv, kvpitch, n0, wave * T::VDMA_PER_WAVE + i, lane);
    issue(0, 0);
  }

  // K^T operand (B of S = Q K^T) in VGPRs
  bf16x8 kf[kKK];
  {
    const int64_t off = ((int64_t)(ck + kj) * p.Hkv + g) * kD + 8 * half;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) kf[kk] = as_bf16x8(kvalid ? ld16(p.k + off + 16 * kk) : zero_u4());
    settle(kf);
  }
  // addresses of this lane's V row (key wave * 32 + col of the block) in LDS
  uint32_t vrow[8];
  {
    const int vr = wave * 32 + col;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) vrow[kk] = T::VBASE + vr * T::ROW + (((2 * kk + half) ^ swz<kD>(vr)) << 4);
  }
  OperandOffsets<kD> off;
  operand_offsets<kD>(off, lane);

  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  acc_fence(dk);
  acc_fence(dv);
  const float c = p.scale_log2;
  // query rows rlo .. rhi see this lane's key
  const int rlo = (BAND && p.wr >= 0) ? kj - (Lk - Lq) - p.wr : INT_MIN / 2;
  const int rhi = (BAND && p.wl >= 0) ? kj - (Lk - Lq) + p.wl : INT_MAX / 2;

  // One barrier per step: after it, stage it (whose copies are the only ones in
  // flight) is in LDS for every wave, and every wave is done with step it - 1,
  // whose buffer then takes the copies of stage it + 1.
  auto stage_in = [&](int it) {
    wait_vmcnt<0>();
    lds_barrier();
    if (it + 1 < total) issue(it + 1, (it + 1) & 1);
  };
  // Per query head of the split: masked steps, unmasked steps, masked steps
  // (separate loops, so the accumulators keep their registers). `it` counts
  // steps over all heads for the copy pipeline.
  int it = 0;
  auto step = [&](int st, auto masked) {
    stage_in(it);
    const int m0 = (sfirst + st) * T::BMQ;
    const lds_char* stg = lds + (it & 1) * T::STAGE;
    const float* f32 = reinterpret_cast<const float*>(smem) + (T::F32 + (it & 1) * T::F32_STAGE) / 4;
    dkdv256_step<decltype(masked)::value, LEFT>(lds, stg, stg + T::TILE, f32, f32 + 64, kf, vrow, dk, dv, c, rlo - m0,
                                          rhi - m0, off, half);
    ++it;
  };
  for (int hg = 0; hg < (total > 0 ? hper : 0); ++hg) {
    for (int st = 0; st < s_full_lo; ++st) step(st, std::true_type());
    for (int st = s_full_lo; st < s_full_hi; ++st) step(st, std::false_type());
    for (int st = s_full_hi; st < nsteps; ++st) step(st, std::true_type());
  }

  acc_fence(dk);
  acc_fence(dv);
  if (kvalid) {
    const int64_t row = ((int64_t)(ck + kj) * p.Hkv + g) * kD + 4 * half;
    if (S == 1) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        store_acc_row(p.dk + row + db * 32, dk[db], p.scale);
        store_acc_row(p.dv + row + db * 32, dv[db], 1.f);
      }
    } else {
      const int64_t part = (int64_t)split * p.total_k * p.Hkv * kD;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        store_acc_row_f32(p.part_dk + part + row + db * 32, dk[db]);
        store_acc_row_f32(p.part_dv + part + row + db * 32, dv[db]);
      }
    }
  }
}

// dK = scale * sum_s part_dk[s], dV = sum_s part_dv[s], in split order; 8
// consecutive values per thread.
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part_dk,
                                                              const float* __restrict__ part_dv,
                                                              uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                              int64_t n8, int splits, float scale) {
  const int64_t plane = n8 * 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const float4* pk = reinterpret_cast<const float4*>(part_dk + s * plane + 8 * i);
      const float4* pv = reinterpret_cast<const float4*>(part_dv + s * plane + 8 * i);
      const float4 k0 = pk[0], k1 = pk[1], v0 = pv[0], v1 = pv[1];
      a[0] += k0.x; a[1] += k0.y; a[2] += k0.z; a[3] += k0.w;
      a[4] += k1.x; a[5] += k1.y; a[6] += k1.z; a[7] += k1.w;
      v[0] += v0.x; v[1] += v0.y; v[2] += v0.z; v[3] += v0.w;
      v[4] += v1.x; v[5] += v1.y; v[6] += v1.z; v[7] += v1.w;
    }
    uint4 ok, ov;
    ok.x = pack_bf16x2(a[0] * scale, a[1] * scale);
    ok.y = pack_bf16x2(a[2] * scale, a[3] * scale);
    ok.z = pack_bf16x2(a[4] * scale, a[5] * scale);
    ok.w = pack_bf16x2(a[6] * scale, a[7] * scale);
    ov.x = pack_bf16x2(v[0], v[1]);
    ov.y = pack_bf16x2(v[2], v[3]);
    ov.z = pack_bf16x2(v[4], v[5]);
    ov.w = pack_bf16x2(v[6], v[7]);
    st16(dk + 8 * i, ok);
    st16(dv + 8 * i, ov);
  }
}


// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

struct Dq256 {
  static constexpr int NT = 256;
  static constexpr int BM = 128;  // query rows x heads per workgroup (32 rows per wave)
  static constexpr int BN = 32;   // keys per tile
  static_assert(BM == kQueryBlock && BN == key_tile(kD), "tile shapes of the host-side plan");
  using KV = RowTile<kD, BN>;
  static constexpr int ROW = KV::ROW;
  static constexpr int TILE = KV::BYTES;  // 16 KB
  static constexpr int STAGE = 2 * TILE;  // K tile, then V tile
  static constexpr size_t LDS_BYTES = 2 * STAGE;
  static constexpr int DMA_PER_WAVE = 2 * KV::DMAS / 4;
  static constexpr int PF = 2;
  static constexpr int RV = 3;
  static_assert(LDS_BYTES <= 65536, "tile offsets must fit the 16-bit LDS immediate");
};

__device__ __forceinline__ void issue_kv_dq256(uint32_t stage, const i32x4& rk, const i32x4& rv, uint32_t pitch,
                                               int n0, int wave, int lane) {
  using T = Dq256;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;
    const bool is_v = qd >= T::KV::DMAS;
    tile_dma<kD, T::BN>(stage + (is_v ? T::TILE : 0), is_v ? rv : rk, pitch, n0, is_v ? qd - T::KV::DMAS : qd, lane);
  }
}

// One 32-key tile: S^T = K Q^T and dP^T = V dO^T (two chains), dS, then
// dQ^T += K^T dS^T one (k-step, head-dim block) unit at a time.
// Keys klo .. khi - 1 are visible to this lane's query row.
template <bool MASK, bool LEFT>
__device__ __forceinline__ void dq256_tile(const lds_char* Ks, const lds_char* Vs, const bf16x8* qf,
                                           const bf16x8* df, f32x16 (&dq)[kDB], float c, float lse2, float dlt,
                                           int n0, int klo, int khi, const OperandOffsets<kD>& off, int half) {
  using T = Dq256;
  constexpr int PF = T::PF, RV = T::RV;
  f32x16 s, dp;
  uint4 fr[PF + 1][2];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    fr[kk][0] = lds_ld16(Ks + off.row(kk));
    fr[kk][1] = lds_ld16(Vs + off.row(kk));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    if (kk + PF < kKK) {
      fr[(kk + PF) % (PF + 1)][0] = lds_ld16(Ks + off.row(kk + PF));
      fr[(kk + PF) % (PF + 1)][1] = lds_ld16(Vs + off.row(kk + PF));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kk == 0) {
      mfma_vgpr0(s, as_bf16x8(fr[0][0]), qf[0]);
      mfma_vgpr0(dp, as_bf16x8(fr[0][1]), df[0]);
    } else {
      mfma_vgpr(s, as_bf16x8(fr[kk % (PF + 1)][0]), qf[kk]);
      mfma_vgpr(dp, as_bf16x8(fr[kk % (PF + 1)][1]), df[kk]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  vgpr_fence(s, dp);
  bf16x8 ka[RV];
#pragma unroll
  for (int u = 0; u < RV - 1; ++u) ka[u] = tr_operand<kD>(Ks + 16 * (u / kDB) * T::ROW, off, u % kDB);
  __builtin_amdgcn_sched_barrier(0);
  float dsv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float pe = fast_exp2(__builtin_fmaf(s[v], c, -lse2));
    if (MASK) {
      const int key = n0 + 16 * (v >> 3) + 8 * half + (v & 7);
      pe = ((!LEFT || key >= klo) && key < khi) ? pe : 0.f;
    }
    dsv[v] = pe * (dp[v] - dlt);
  }
  bf16x8 sb;
#pragma unroll
  for (int u = 0; u < 2 * kDB; ++u) {
    const int ks = u / kDB, db = u % kDB;
    if (u + RV - 1 < 2 * kDB) {
      const int w = u + RV - 1;
      ka[w % RV] = tr_operand<kD>(Ks + 16 * (w / kDB) * T::ROW, off, w % kDB);
    }
    if (db == 0)
      sb = to_bf16x8(dsv[8 * ks + 0], dsv[8 * ks + 1], dsv[8 * ks + 2], dsv[8 * ks + 3], dsv[8 * ks + 4],
                     dsv[8 * ks + 5], dsv[8 * ks + 6], dsv[8 * ks + 7]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_agpr(dq[db], ka[u % RV], sb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// LEFT: the band has a left bound (window_left >= 0); without one, a row's
// visible keys start at key 0 and masked tiles test only their upper bound.
template <bool BAND, bool LEFT>
__global__ __launch_bounds__(256, 1) void bwd_dq256_kernel(BwdParams p) {
  using T = Dq256;
  extern __shared__ __align__(16) uint16_t smem[];
  lds_char* lds = (lds_char*)smem;

  // the workgroup covers hw heads of one KV group, bm rows of each (as the forward)
  const int r = p.Hq / p.Hkv;
  const int hw = block_heads(r), hwl = log2_small(hw), bm = T::BM / hw;
  const int64_t L = xcd_logical(blockIdx.x, r >> hwl);
  const int heads = p.Hq >> hwl;
  const int rank = (int)(L / heads);
  const int hs = (int)(L % heads);
  Item item;
  if (!decode_item<false>(p.cu_q, p.cu_k, p.num_seqs, bm, p.levels, rank, item)) return;
  const int g = (hs << hwl) / r;
  const int mblk = item.m, cq = item.cq, Lq = item.Lq, ck = item.ck, Lk = item.Lk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int h = (hs << hwl) + (wave & (hw - 1));
  // query blocks aligned toward the end of the sequence, as in the forward
  const int q0 = mblk * bm - query_lead(Lq, bm, T::BN);
  const int qi = q0 + (wave >> hwl) * 32 + col;
  const bool qvalid = qi >= 0 && qi < Lq;
  const int qa = qvalid ? qi : 0;  // a valid row for address arithmetic

  // key tiles [t_lo, t_hi), the unmasked ones [f_lo, f_hi)
  int t_lo = 0, t_hi = ceil_div(Lk, T::BN), f_lo = 0, f_hi = Lk / T::BN;
  if (BAND) {
    const TileSpan ts = key_tiles(max(q0, 0), min(q0 + bm, Lq) - 1, T::BN, Lq, Lk, p.wl, p.wr);
    t_lo = ts.lo;
    t_hi = ts.hi;
    f_lo = ts.full_lo;
    f_hi = max(f_lo, ts.full_hi);
  }
  const int klo = BAND ? band_lo(qi, Lq, Lk, p.wl) : 0;
  const int khi = BAND ? band_hi(qi, Lq, Lk, p.wr) : Lk;

  const uint32_t pitch = (uint32_t)p.Hkv * kD * 2;
  const int64_t kvoff = ((int64_t)ck * p.Hkv + g) * kD;
  const i32x4 rk = head_rows_rsrc<kD>(p.k + kvoff, Lk, pitch);
  const i32x4 rv = head_rows_rsrc<kD>(p.v + kvoff, Lk, pitch);
  const uint32_t lds0 = lds_addr(lds);
  if (t_hi > t_lo) issue_kv_dq256(lds0 + (t_lo & 1) * T::STAGE, rk, rv, pitch, t_lo * T::BN, wave, lane);

  bf16x8 qf[kKK], df[kKK];
  {
    const int64_t off = ((int64_t)(cq + qa) * p.Hq + h) * kD + 8 * half;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qf[kk] = as_bf16x8(qvalid ? ld16(p.q + off + 16 * kk) : zero_u4());
      df[kk] = as_bf16x8(qvalid ? ld16(p.dout + off + 16 * kk) : zero_u4());
    }
  }
  settle(qf);
  settle(df);
  const int64_t lidx = (int64_t)h * p.total_q + cq + qa;
  float lse2 = qvalid ? p.lse2[lidx] : INFINITY;
  float dlt = qvalid ? p.delta[lidx] : 0.f;
  asm volatile("" : "+v"(lse2), "+v"(dlt));
  OperandOffsets<kD> off;
  operand_offsets<kD>(off, lane);

  f32x16 dq[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dq[db] = zero16();
  acc_fence(dq);
  const float c = p.scale_log2;

  // one barrier per tile: stage n has landed for every wave, and every wave is
  // done with tile n - 1, whose buffer then takes the copies of tile n + 1
  auto stage_in = [&](int n) {
    wait_vmcnt<0>();
    lds_barrier();
    if (n + 1 < t_hi) issue_kv_dq256(lds0 + ((n + 1) & 1) * T::STAGE, rk, rv, pitch, (n + 1) * T::BN, wave, lane);
  };
  auto tile = [&](int n, auto masked) {
    stage_in(n);
    const lds_char* cur = lds + (n & 1) * T::STAGE;
    dq256_tile<decltype(masked)::value, LEFT>(cur, cur + T::TILE, qf, df, dq, c, lse2, dlt, n * T::BN, klo, khi, off, half);
  };
  for (int n = t_lo; n < f_lo; ++n) tile(n, std::true_type());
  for (int n = f_lo; n < f_hi; ++n) tile(n, std::false_type());
  for (int n = f_hi; n < t_hi; ++n) tile(n, std::true_type());

  acc_fence(dq);
  if (qvalid) {
    uint16_t* row = p.dq + ((int64_t)(cq + qi) * p.Hq + h) * kD + 4 * half;
#pragma unroll
    for (int db = 0; db < kDB; ++db) store_acc_row(row + db * 32, dq[db], p.scale);
  }
}

template <bool BAND, bool LEFT>
hipError_t launch_main_t(const BwdArgs& a, float* lse2, float* part_dk, float* part_dv, int splits) {
  const FwdArgs& f = a.f;
  hipStream_t stream = (hipStream_t)f.stream;
  BwdParams p;
  p.ds = nullptr;  // the stored-dS path is for head dims 64 / 128
  p.ds_pitch = 0;
  p.q = static_cast<const uint16_t*>(f.q);
  p.k = static_cast<const uint16_t*>(f.k);
  p.v = static_cast<const uint16_t*>(f.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.delta = a.delta;
  p.lse2 = lse2;
  p.out = static_cast<const uint16_t*>(a.out);
  p.lse = a.lse;
  p.cu_q = f.cu_q;
  p.cu_k = f.cu_k;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.part_dk = part_dk;
  p.part_dv = part_dv;
  p.num_seqs = f.num_seqs;
  p.total_q = (int)f.total_q;
  p.total_k = (int)f.total_k;
  p.Hq = f.Hq;
  p.Hkv = f.Hkv;
  p.splits = splits;
  const Band bd = band_of(f);
  p.wl = bd.wl;
  p.wr = bd.wr;
  p.scale = f.scale;
  p.scale_log2 = f.scale * kLog2e;

  if (f.total_k > 0) {
    using T = Dkdv256;
    auto kern = bwd_dkdv256_kernel<BAND, LEFT>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    BwdParams pk = p;
    pk.levels = ceil_div(f.max_k, T::BNK);
    const int64_t grid = grid_for(f.total_k, f.num_seqs, pk.levels, T::BNK, f.Hkv * splits, splits);
    if (grid > 0 && pk.levels > 0) {
      prof_begin("attn_bwd_dkdv", stream);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, pk);
      prof_end(stream);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (splits > 1) {
      e = launch_dkdv_reduce(part_dk, part_dv, p.dk, p.dv, f.total_k * f.Hkv * kD / 8, splits, f.scale, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (f.total_q > 0) {
    using T = Dq256;
    auto kern = bwd_dq256_kernel<BAND, LEFT>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    BwdParams pq = p;
    const int hw = block_heads(f.Hq / f.Hkv), hwl = log2_small(hw), bm = T::BM / hw;
    pq.levels = ceil_div(f.max_q, bm);
    const int64_t grid = grid_for(f.total_q, f.num_seqs, pq.levels, bm, f.Hq >> hwl, (f.Hq / f.Hkv) >> hwl);
    if (grid > 0 && pq.levels > 0) {
      prof_begin("attn_bwd_dq", stream);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, pq);
      prof_end(stream);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

// The ordered reduce of split partial sums, for any head dim (n8: elements / 8).
hipError_t launch_dkdv_reduce(const float* part_dk, const float* part_dv, uint16_t* dk, uint16_t* dv, int64_t n8,
                              int splits, float scale, hipStream_t stream) {
  if (n8 <= 0) return hipSuccess;
  int64_t rgrid = (n8 + 255) / 256;
  if (rgrid > 8192) rgrid = 8192;
  prof_begin("attn_bwd_dkdv_reduce", stream);
  hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3((unsigned)rgrid), dim3(256), 0, stream, part_dk, part_dv, dk, dv,
                     n8, splits, scale);
  prof_end(stream);
  return hipGetLastError();
}

hipError_t launch_bwd_main_d256(const BwdArgs& a, float* lse2, float* part_dk, float* part_dv, int splits) {
  const Band bd = band_of(a.f);
  if (!bd.band) return launch_main_t<false, false>(a, lse2, part_dk, part_dv, splits);
  return bd.wl >= 0 ? launch_main_t<true, true>(a, lse2, part_dk, part_dv, splits)
                    : launch_main_t<true, false>(a, lse2, part_dk, part_dv, splits);
}

}  // namespace av
