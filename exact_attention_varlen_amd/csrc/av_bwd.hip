// av_bwd.hip — backward kernels: gradients of sum(dout * out) for exact varlen
// GQA attention, deterministic (no atomics, every sum in a fixed order).
//
// The FlashAttention repository guide (Backward Kernels) splits the backward
// into a preprocess kernel, a main kernel and a postprocess kernel. Here:
//  1. row terms        per query row and head: Delta_i = sum_d dO_id * O_id
//                       (fp32) and the LSE in base 2, lse2_i = lse_i * log2(e)
//                       (+inf for rows without a visible key, so that
//                       exp2(s - lse2) is exactly 0 there), into the caller's
//                       workspace: at head dims 64 / 128 by the dQ kernel (3),
//                       which holds the row's dO anyway and runs first; at head
//                       dim 256 by bwd_prep_kernel.
//  2. bwd_dkdv_kernel   key-stationary: a workgroup owns 128 keys of one KV head
//                       and loops over every query head of that head's group and
//                       every 64-row query block that can see the keys,
//                       recomputing P from the LSE:
//                         S = Q K^T, P = exp2(S * scale * log2 e - lse2),
//                         dP = dO V^T, dS = P * (dP - Delta),
//                         dV += P^T dO, dK += dS^T Q.
//                       The sum over the group's query heads happens in fp32
//                       registers in a fixed order: no atomics, no scratch.
//  3. bwd_dq_kernel     query-stationary: a workgroup owns 32 query rows per
//                       wave, of hw = block_heads(group size) query heads of one
//                       KV group (128 / hw rows of each), and loops over the
//                       visible 64-key tiles in ascending order: dQ += dS K.
// dQ and dK are scaled by softmax_scale at the end. Head dim 256 uses the
// main kernels of av_bwd_d256.hip after the same preprocess.
//
// gfx950 mapping (as in the forward): Q/dO tiles (dK/dV kernel) and K/V tiles
// (dQ kernel) go HBM -> LDS by range-checked buffer-load DMA, double-buffered,
// XOR-swizzled; the operands that contract over rows (Q^T, dO^T, K^T) are read
// with ds_read_b64_tr_b16 from the row-major tiles; all products are
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "av_bwd.h"
#include "av_common.h"
#include "av_launch.h"
#include "av_tiles.h"

namespace av {

hipError_t launch_bwd_main_d256(const BwdArgs& a, float* lse2, float* part_dk, float* part_dv,
                                int splits);  // av_bwd_d256.hip
hipError_t launch_dkdv_reduce(const float* part_dk, const float* part_dv, uint16_t* dk, uint16_t* dv, int64_t n8,
                              int splits, float scale, hipStream_t stream);  // av_bwd_d256.hip

size_t bwd_workspace_bytes(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D) {
  return bwd_ws_bytes_for(total_q, total_k, Hq, Hkv, D, dkdv_splits(total_k, Hq, Hkv, D));
}

size_t bwd_min_workspace_bytes(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D) {
  return bwd_ws_bytes_for(total_q, total_k, Hq, Hkv, D, 1);
}

size_t bwd_ds_workspace_bytes(int64_t total_q, int64_t total_k, int max_q, int max_k, int Hq, int Hkv, int D) {
  const size_t ds = ds_buffer_bytes(total_q, total_k, max_q, max_k, Hq, D);
  return ds ? bwd_workspace_bytes(total_q, total_k, Hq, Hkv, D) + ds : 0;
}

int bwd_ds_pitch(int max_q) { return ds_pitch_of(max_q); }

// ---------------------------------------------------------------------------
// 1. preprocess
// ---------------------------------------------------------------------------

__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
  float acc = 0.f;
  acc += bf16_lo(a.x) * bf16_lo(b.x);
  acc += bf16_hi(a.x) * bf16_hi(b.x);
  acc += bf16_lo(a.y) * bf16_lo(b.y);
  acc += bf16_hi(a.y) * bf16_hi(b.y);
  acc += bf16_lo(a.z) * bf16_lo(b.z);
  acc += bf16_hi(a.z) * bf16_hi(b.z);
  acc += bf16_lo(a.w) * bf16_lo(b.w);
  acc += bf16_hi(a.w) * bf16_hi(b.w);
  return acc;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ dout,
                                                       const uint16_t* __restrict__ out, const float* __restrict__ lse,
                                                       float* __restrict__ delta, float* __restrict__ lse2,
                                                       int total_q, int Hq) {
  constexpr int LPR = D / 8;      // lanes per (row, head)
  constexpr int RPB = 256 / LPR;  // (row, head) pairs per workgroup pass
  const int64_t nrows = (int64_t)total_q * Hq;
  const int sub = threadIdx.x % LPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; row < nrows; row += (int64_t)gridDim.x * RPB) {
    const uint4 a = ld16(dout + row * D + sub * 8);
    const uint4 b = ld16(out + row * D + sub * 8);
    float acc = dot8_bf16(a, b);
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (sub == 0) {
      const int i = (int)(row / Hq);
      const int h = (int)(row - (int64_t)i * Hq);
      const int64_t idx = (int64_t)h * total_q + i;
      delta[idx] = acc;
      const float l = lse[idx];
      lse2[idx] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. key-stationary dK / dV
// ---------------------------------------------------------------------------

template <int D>
struct DkdvCfg {
  static constexpr int NT = 256;
  static constexpr int BNK = 128;                 // keys per workgroup (32 per wave)
  static constexpr int BMQ = (D <= 128) ? 128 : 64;  // query rows per step
  using QT = RowTile<D, BMQ>;
  static constexpr int ROW = QT::ROW;
  static constexpr int TILE = QT::BYTES;
  static constexpr int F32 = 2 * TILE;            // lse2[BMQ] then Delta[BMQ]
  static constexpr int STAGE = 2 * TILE + 8 * BMQ;
  static constexpr size_t LDS_BYTES = 2 * STAGE;
  static constexpr int DMA_PER_WAVE = 2 * QT::DMAS / 4;  // Q and dO copies
  static constexpr int F32_DMAS = BMQ / 64;              // 64-row fp32 copies per array
  static_assert(D > 128 || (BNK == kKeyBlock && BMQ == query_step(D)), "tile shapes of the host-side plan");
};

template <int D>
__device__ __forceinline__ void issue_qdo(uint32_t stage, const i32x4& rq, const i32x4& rdo, const i32x4& rl,
                                          const i32x4& rd, uint32_t pitch, int m0, int wave, int lane) {
  using T = DkdvCfg<D>;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;
    const bool is_do = qd >= T::QT::DMAS;
    tile_dma<D, T::BMQ>(stage + (is_do ? T::TILE : 0), is_do ? rdo : rq, pitch, m0, is_do ? qd - T::QT::DMAS : qd,
                        lane);
  }
  // lse2 rows on wave 0, Delta rows on wave 1 (64 rows per copy)
#pragma unroll
  for (int j = 0; j < T::F32_DMAS; ++j) {
    if (wave == 0) rows64_f32_dma(stage + T::F32 + 256 * j, rl, m0 + 64 * j, lane);
    if (wave == 1) rows64_f32_dma(stage + T::F32 + 4 * T::BMQ + 256 * j, rd, m0 + 64 * j, lane);
  }
}

// S / dP products of the dK / dV kernel, written as asm so that their
// accumulators are VGPRs, which the VALU reads next, and the K / V operand is an
// AGPR. (At one wave per SIMD the compiler gives every MFMA an AGPR result, and
// each score then costs a v_accvgpr_read before the VALU can use it.) The asm is
// opaque to the compiler's hazard checks: s_fence_scores() gives the results the
// wait states they need before any VALU instruction reads them, and has them as
// operands so that no read moves above it. The A operand comes from an LDS read
// (the compiler's s_waitcnt covers it), the B operand from a global load at the
// start of the item.
__device__ __forceinline__ void mfma_score0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_score(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void s_fence_scores(f32x16& s, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s), "+v"(d));
}

// Scheduling hints (instruction classes for __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedValu = 0x002;

// One step: BMQ query rows (starting at sequence row m0) against this wave's
// 32 keys, as NB blocks of 32 query rows. Each block b needs
//   A(b): S = Q K^T and dP = dO V^T (2 KK MFMAs, Q / dO rows from LDS),
//   B(b): P = exp2(S c - lse2) (masked), dS = P (dP - Delta), packed to bf16,
//         for its two 16-query k-steps (8 scores per lane each),
//   C(b): dV += P^T dO and dK += dS^T Q (4 DB MFMAs, transposed rows from LDS).
// The matrix core runs one MFMA at a time and a wave issues in order, so the
// vector work of B only overlaps the MFMAs when it is spread between them. The
// step is software-pipelined over the blocks in phases of NU = 2 KK = 4 DB MFMA
// units each:
//   X(b): A(b)     with B(b - 1, k-step 1) between its MFMAs,
//   Y(b): C(b - 1) with B(b, k-step 0) between its MFMAs,
// for b = 0 .. NB. X(0) has no B part and X(NB) no A part, Y(0) no C part and
// Y(NB) no B part; so that no phase is left with vector work alone, X(NB) also
// runs the first units of C(NB - 1) and Y(0) the first units of A(1). Each
// unit also issues the LDS reads one or two units ahead: the next k-steps of
// the Q / dO rows and the transposed operands of C (a ring of RV). The rows'
// lse2 / Delta of a B part are read at the start of the phase before the one
// that uses them (their registers are free by then), a whole phase ahead.
// STORE: the first two units of Y(b) also write dS of block b - 1 (16 bytes per
// lane and k-step: this lane's key, 8 consecutive query rows) to the stored-dS
// row `dsrow` (this lane's key, query row m0 + 8 half), for the dQ kernel.
// x0(u) runs in unit u of X(0), whose MFMAs have no vector work beside them:
// the kernel issues the next stage's copies there.
template <int D, bool MASK, bool LEFT, bool STORE, class X0>
__device__ __forceinline__ void dkdv_step(const lds_char* Qs, const lds_char* dOs, const float* lse2_s,
                                          const float* dlt_s, const bf16x8* kf, const bf16x8* vf, f32x16* dk,
                                          f32x16* dv, float c, int m0, int rlo, int rhi, const OperandOffsets<D>& off,
                                          int half, uint16_t* dsrow, bool kvalid, const X0& x0) {
  using T = DkdvCfg<D>;
  constexpr int KK = D / 16, DB = D / 32, NB = T::BMQ / 32, PF = 2, RV = 3;
  constexpr int NU = 2 * KK;  // MFMA units per phase
  static_assert(NU == 4 * DB, "the units of A(b) and C(b) must pair up");
  const int rl = rlo - m0, rh = rhi - m0;  // step-relative rows that see this lane's key

  f32x16 sacc[2], dacc[2];          // S and dP of block b in [b & 1]
  uint32_t pw[2][2][4], sw[2][2][4];  // bf16 pairs of P and dS: [b & 1][k-step][pair]
  float l2[2][8], dl[2][8];         // lse2 / Delta of the rows of B(., k-step)
  float pe[8], pm[8], dsv[8];
  uint4 fr[PF + 1][2];              // Q / dO row operands of A, PF k-steps ahead
  bf16x8 va[RV];                    // transposed operands of C, RV - 1 units ahead

  auto load_rowvals = [&](int b, int ks) {
    const int qo = 32 * b + 16 * ks + 8 * half;
    const float4 a0 = *reinterpret_cast<const float4*>(lse2_s + qo);
    const float4 a1 = *reinterpret_cast<const float4*>(lse2_s + qo + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(dlt_s + qo);
    const float4 b1 = *reinterpret_cast<const float4*>(dlt_s + qo + 4);
    l2[ks][0] = a0.x; l2[ks][1] = a0.y; l2[ks][2] = a0.z; l2[ks][3] = a0.w;
    l2[ks][4] = a1.x; l2[ks][5] = a1.y; l2[ks][6] = a1.z; l2[ks][7] = a1.w;
    dl[ks][0] = b0.x; dl[ks][1] = b0.y; dl[ks][2] = b0.z; dl[ks][3] = b0.w;
    dl[ks][4] = b1.x; dl[ks][5] = b1.y; dl[ks][6] = b1.z; dl[ks][7] = b1.w;
  };
  auto load_rows = [&](int b, int kk) {
    fr[kk % (PF + 1)][0] = lds_ld16(Qs + 32 * b * T::ROW + off.row(kk));
    fr[kk % (PF + 1)][1] = lds_ld16(dOs + 32 * b * T::ROW + off.row(kk));
  };
  // unit w of C(b): k-step w / (2 DB), head-dim block (w / 2) % DB, dV (even) or dK (odd)
  auto load_tr = [&](int b, int w) {
    const int ks = w / (2 * DB), db = (w / 2) % DB;
    const lds_char* rows = ((w & 1) ? Qs : dOs) + (32 * b + 16 * ks) * T::ROW;
    va[w % RV] = tr_operand<D>(rows, off, db);
  };
  // B(b, ks): score e is issued (exp) at unit iss(e) and finished one unit later
  auto b_issue = [&](int b, int ks, int e) {
    pe[e] = fast_exp2(__builtin_fmaf(sacc[b & 1][8 * ks + e], c, -l2[ks][e]));
  };
  auto b_finish = [&](int b, int ks, int e) {
    float pv = pe[e];
    if (MASK) {
      const int row = 32 * b + 16 * ks + 8 * half + e;
      pv = (row >= rl && (!LEFT || row <= rh)) ? pv : 0.f;
    }
    pm[e] = pv;
    dsv[e] = pv * (dacc[b & 1][8 * ks + e] - dl[ks][e]);
    if (e & 1) {
      pw[b & 1][ks][e >> 1] = pack_bf16x2(pm[e - 1], pm[e]);
      sw[b & 1][ks][e >> 1] = pack_bf16x2(dsv[e - 1], dsv[e]);
    }
  };
  // the B share of unit u: issue the scores whose slot is u, finish those of u - 1
  auto b_share = [&](int b, int ks, int u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e * NU / 8 == u) b_issue(b, ks, e);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e * NU / 8 + 1 == u) b_finish(b, ks, e);
    }
  };
  auto b_tail = [&](int b, int ks) {  // scores whose finishing slot is past the phase
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e * NU / 8 + 1 >= NU) b_finish(b, ks, e);
    }
  };
  // unit w of C(b): dV (w even) or dK (w odd) of head-dim block (w / 2) % DB and
  // k-step w / (2 DB), its transposed operand from the ring
  auto c_unit = [&](int b, int w) {
    const int ks = w / (2 * DB), db = (w / 2) % DB;
    const uint32_t* wv = (w & 1) ? sw[b & 1][ks] : pw[b & 1][ks];
    const bf16x8 bop = as_bf16x8(make_uint4(wv[0], wv[1], wv[2], wv[3]));
    f32x16& acc = (w & 1) ? dk[db] : dv[db];
    acc = mfma32x32x16(va[w % RV], bop, acc);
  };
  // X(NB) has no A MFMAs of its own: it runs the first CX units of C(NB - 1),
  // which need only k-step 0's P / dS (formed in Y(NB - 1)), one every other
  // unit from unit 2 on, between the vector work of B(NB - 1, 1); Y(NB) runs the
  // rest. The ring of C(NB - 1) is warmed at the start of X(NB).
  constexpr int CX = (NU / 2 - 1 < 2 * DB) ? NU / 2 - 1 : 2 * DB;
  // unit v of A(b): S (v even) or dP (v odd) for k-step v / 2, fetching the
  // Q / dO rows of k-step v / 2 + PF first
  auto a_unit = [&](int b, int v) {
    const int kk = v / 2, j = v & 1;
    if (j == 0 && kk + PF < KK) load_rows(b, kk + PF);
    f32x16& acc = j ? dacc[b & 1] : sacc[b & 1];
    if (kk == 0)
      mfma_score0(acc, as_bf16x8(fr[kk % (PF + 1)][j]), j ? vf[kk] : kf[kk]);
    else
      mfma_score(acc, as_bf16x8(fr[kk % (PF + 1)][j]), j ? vf[kk] : kf[kk]);
  };
  // Likewise Y(0) has no C MFMAs: it runs the first AY units of A(1), one every
  // other unit from unit 2 on, and X(1) the rest (every other unit, and the last
  // unit). Block 1's first rows are fetched at the end of X(0).
  constexpr int AY = NU / 2 - 1;
  static_assert(NB >= 2, "the head start of A(1) needs a second block");

#pragma unroll
  for (int kk = 0; kk < PF; ++kk) load_rows(0, kk);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b <= NB; ++b) {
    // ---- X(b): A(b), B(b - 1, 1) ----
    if (b < NB) load_rowvals(b, 0);  // lse2 / Delta of B(b, 0), a phase ahead
    if (b == NB) {
#pragma unroll
      for (int w = 0; w < RV - 1; ++w) load_tr(b - 1, w);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int kk = u / 2, j = u & 1;
      if (b < NB && b != 1) a_unit(b, u);
      if (b == 0) x0(u);  // the caller's work for unit u of X(0) (the next stage's copies)
      if (b == 1) {
        const int v = (j == 0) ? AY + kk : (u == NU - 1 ? NU - 1 : -1);
        if (v >= 0) a_unit(1, v);
      }
      if (b == NB && u >= 2 && j == 0 && kk - 1 < CX) {
        if (kk - 1 + RV - 1 < NU) load_tr(b - 1, kk - 1 + RV - 1);
        c_unit(b - 1, kk - 1);
      }
      if (b >= 1) b_share(b - 1, 1, u);
      // warm the ring of C(b - 1) in the last units
      if (b >= 1 && b < NB && u >= NU - (RV - 1)) load_tr(b - 1, u - (NU - (RV - 1)));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (b == 0) {
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) load_rows(1, kk);
    }
    if (b < NB) s_fence_scores(sacc[b & 1], dacc[b & 1]);
    if (b >= 1) b_tail(b - 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    // ---- Y(b): C(b - 1), B(b, 0) ----
    if (b < NB) load_rowvals(b, 1);  // lse2 / Delta of B(b, 1), a phase ahead
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (STORE && b >= 1 && u < 2 && kvalid) {
        const uint32_t* w = sw[(b - 1) & 1][u];
        *reinterpret_cast<uint4*>(dsrow + 32 * (b - 1) + 16 * u) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      if (b >= 1) {
        const int w = (b == NB) ? u + CX : u;  // C(NB - 1)'s first CX units ran in X(NB)
        if (w < NU) {
          if (w + RV - 1 < NU) load_tr(b - 1, w + RV - 1);
          c_unit(b - 1, w);
        }
      }
      if (b == 0 && u >= 2 && (u & 1) == 0 && u / 2 - 1 < AY) a_unit(1, u / 2 - 1);
      if (b < NB) b_share(b, 0, u);
      // the first Q / dO row k-steps of the next block (block 1's: end of X(0))
      if (b >= 1 && b + 1 < NB && u >= NU - PF) load_rows(b + 1, u - (NU - PF));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (b < NB) b_tail(b, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// BAND: the visible keys of a row form a band (causal and / or a local window).
// LEFT: the band has a left bound (window_left >= 0). Without one, every row
// past a key's first visible row sees it, and masked steps test that bound only.
// STORE: also write dS to the stored-dS buffer p.ds (bwd_dq_ds_kernel reads it).
// SPLIT: the item covers r / p.splits query heads of the group (split `split`)
// and writes fp32 partial dK / dV sums (p.part_dk / part_dv, plane `split`), which
// bwd_dkdv_reduce_kernel adds in split order.
template <int D, bool BAND, bool LEFT, bool STORE, bool SPLIT = false>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  static_assert(!(SPLIT && STORE), "the stored-dS path runs without splits");
  using T = DkdvCfg<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  lds_char* lds = (lds_char*)smem;

  // work item: (sequence, key block) ranked by descending work, x KV heads (x
  // query-head splits, innermost, as in the head_dim 256 kernel). The rank's
  // level counts key blocks from the end of the sequence, so the blocks seen by
  // the most query rows come first.
  int rank, g, split = 0;
  if constexpr (SPLIT) {
    const int64_t L = blockIdx.x;
    const int64_t per = (int64_t)p.Hkv * p.splits;
    rank = (int)(L / per);
    const int rem = (int)(L % per);
    g = rem / p.splits;
    split = rem % p.splits;
  } else {
    const int64_t L = xcd_logical(blockIdx.x, 1);
    rank = (int)(L / p.Hkv);
    g = (int)(L % p.Hkv);
  }
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
  const int nh = SPLIT ? r / p.splits : r;             // query heads of this item
  const int h0 = SPLIT ? g * r + split * nh : g * r;   // the first of them

  // query steps [sfirst, sfirst + nsteps) whose rows see a key of this block,
  // and among them the unmasked ones [s_full_lo, s_full_hi): every row sees
  // every key of the block (rows past Lq read as zero and add nothing)
  int sfirst = 0, nsteps = ceil_div(Lq, T::BMQ), s_full_lo = 0, s_full_hi = nsteps;
  if (BAND) {
    const TileSpan ts = query_steps(n0, min(n0 + T::BNK, Lk) - 1, T::BMQ, Lq, Lk, p.wl, p.wr);
    sfirst = ts.lo;
    nsteps = ts.hi - ts.lo;
    s_full_lo = ts.full_lo - sfirst;
    s_full_hi = ts.full_hi - sfirst;
  }
  const int total = (nsteps > 0) ? nsteps * nh : 0;

  const uint32_t pitch = (uint32_t)p.Hq * D * 2;
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int it, uint32_t stage) {
    const int h = h0 + it / nsteps;
    const int m0 = (sfirst + it % nsteps) * T::BMQ;
    const int64_t qoff = ((int64_t)cq * p.Hq + h) * D;
    const i32x4 rq = head_rows_rsrc<D>(p.q + qoff, Lq, pitch);
    const i32x4 rdo = head_rows_rsrc<D>(p.dout + qoff, Lq, pitch);
    const int64_t roff = (int64_t)h * p.total_q + cq;
    const i32x4 rl = make_rsrc(p.lse2 + roff, (uint32_t)Lq * 4u);
    const i32x4 rd = make_rsrc(p.delta + roff, (uint32_t)Lq * 4u);
    issue_qdo<D>(stage, rq, rdo, rl, rd, pitch, m0, wave, lane);
  };
  if (total > 0) issue(0, lds0);

  // K^T and V^T operands (B of S = Q K^T and of dP = dO V^T)
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t off = ((int64_t)(ck + kj) * p.Hkv + g) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = as_bf16x8(kvalid ? ld16(p.k + off + 16 * kk) : zero_u4());
      vf[kk] = as_bf16x8(kvalid ? ld16(p.v + off + 16 * kk) : zero_u4());
    }
    // Consumed here, in AGPRs (the score MFMAs read them from there): the
    // compiler then waits for these loads once, before the step loop. Left
    // pending into the loop, its wait at their first use would also wait for
    // the next stage's Q / dO copies, issued just before, in every step.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+a"(kf[kk]), "+a"(vf[kk]));
  }
  OperandOffsets<D> off;
  operand_offsets<D>(off, lane);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  const float c = p.scale_log2;
  // query rows rlo .. rhi see this lane's key
  const int rlo = (BAND && p.wr >= 0) ? kj - (Lk - Lq) - p.wr : INT_MIN / 2;
  const int rhi = (BAND && p.wl >= 0) ? kj - (Lk - Lq) + p.wl : INT_MAX / 2;

  // Per query head of the group: masked steps (near the band's right edge),
  // unmasked steps, masked steps (near its left edge), as separate loops so the
  // accumulators keep their registers from step to step. `it` counts steps over
  // all heads for the double-buffer and copy pipeline.
  // One barrier per step: after it, stage it (whose copies are the only ones in
  // flight) is in LDS for every wave, and every wave is done with step it - 1,
  // whose buffer then takes the copies of stage it + 1.
  auto stage_in = [&](int it) {
    wait_vmcnt<0>();
    lds_barrier();
  };
  int it = 0;
  // stored dS: this lane's key row of query head g r (the group's first head),
  // at query row 8 half; each head adds a plane of total_k rows, each step m0
  uint16_t* ds_key = nullptr;
  int64_t ds_plane = 0;
  if (STORE) {
    ds_key = p.ds + ((int64_t)g * r * p.total_k + ck + (kvalid ? kj : 0)) * p.ds_pitch + kDsLead + 8 * half;
    ds_plane = (int64_t)p.total_k * p.ds_pitch;
  }
  auto step = [&](int hg, int st, auto masked) {
    stage_in(it);
    const int m0 = (sfirst + st) * T::BMQ;
    const lds_char* stg = lds + (it & 1) * T::STAGE;
    const float* f32 = reinterpret_cast<const float*>(smem) + ((it & 1) * T::STAGE + T::F32) / 4;
    // the copies of stage it + 1, one or two per unit of the step's first phase
    static_assert(T::DMA_PER_WAVE <= D / 8 && T::F32_DMAS <= D / 8, "copies fit the units of X(0)");
    const bool next = it + 1 < total;
    const int h1 = h0 + (it + 1) / nsteps;
    const int m1 = (sfirst + (it + 1) % nsteps) * T::BMQ;
    const int64_t qoff1 = ((int64_t)cq * p.Hq + h1) * D;
    const int64_t roff1 = (int64_t)h1 * p.total_q + cq;
    const uint32_t stage1 = lds0 + ((it + 1) & 1) * T::STAGE;
    auto x0 = [&](int u) {
      if (!next) return;
      if (u < T::DMA_PER_WAVE) {
        const int qd = wave * T::DMA_PER_WAVE + u;
        const bool is_do = qd >= T::QT::DMAS;
        const i32x4 rs = head_rows_rsrc<D>((is_do ? p.dout : p.q) + qoff1, Lq, pitch);
        tile_dma<D, T::BMQ>(stage1 + (is_do ? T::TILE : 0), rs, pitch, m1, is_do ? qd - T::QT::DMAS : qd, lane);
      }
      if (u < T::F32_DMAS && wave < 2) {  // lse2 rows on wave 0, Delta rows on wave 1
        const i32x4 rs = make_rsrc((wave == 0 ? p.lse2 : p.delta) + roff1, (uint32_t)Lq * 4u);
        rows64_f32_dma(stage1 + T::F32 + (wave == 0 ? 0 : 4 * T::BMQ) + 256 * u, rs, m1 + 64 * u, lane);
      }
    };
    dkdv_step<D, decltype(masked)::value, LEFT, STORE>(stg, stg + T::TILE, f32, f32 + T::BMQ, kf, vf, dk, dv, c, m0,
                                                      rlo, rhi, off, half,
                                                      STORE ? ds_key + hg * ds_plane + m0 : nullptr, kvalid, x0);
    ++it;
  };
  for (int hg = 0; hg < (total > 0 ? nh : 0); ++hg) {
    for (int st = 0; st < s_full_lo; ++st) step(hg, st, std::true_type());
    for (int st = s_full_lo; st < s_full_hi; ++st) step(hg, st, std::false_type());
    for (int st = s_full_hi; st < nsteps; ++st) step(hg, st, std::true_type());
  }

  if (kvalid) {
    const int64_t base = ((int64_t)(ck + kj) * p.Hkv + g) * D + 4 * half;
    if constexpr (SPLIT) {
      const int64_t part = (int64_t)split * p.total_k * p.Hkv * D + base;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        store_acc_row_f32(p.part_dk + part + db * 32, dk[db]);
        store_acc_row_f32(p.part_dv + part + db * 32, dv[db]);
      }
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        store_acc_row(p.dk + base + db * 32, dk[db], p.scale);
        store_acc_row(p.dv + base + db * 32, dv[db], 1.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. query-stationary dQ
// ---------------------------------------------------------------------------

template <int D>
struct DqCfg {
  using KV = RowTile<D, 64>;
  static constexpr int NT = 256;
  static constexpr int BM = 128;  // query rows x heads per workgroup (32 rows per wave)
  static constexpr int BN = 64;   // keys per tile
  static constexpr int ROW = KV::ROW;
  static constexpr int TILE = KV::BYTES;
  static constexpr int STAGE = 2 * TILE;
  static constexpr size_t LDS_BYTES = 2 * STAGE;
  static constexpr int DMA_PER_WAVE = 2 * KV::DMAS / 4;
  static constexpr int WAVES_PER_SIMD = (D <= 128) ? 2 : 1;
  static_assert(D > 128 || (BM == kQueryBlock && BN == key_tile(D)), "tile shapes of the host-side plan");
};

template <int D>
__device__ __forceinline__ void issue_kv_dq(uint32_t stage, const i32x4& rk, const i32x4& rv, uint32_t pitch, int n0,
                                           int wave, int lane) {
  using T = DqCfg<D>;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;
    const bool is_v = qd >= T::KV::DMAS;
    tile_dma<D, 64>(stage + (is_v ? T::TILE : 0), is_v ? rv : rk, pitch, n0, is_v ? qd - T::KV::DMAS : qd, lane);
  }
}

// Keys klo .. khi - 1 are visible to this lane's query row (klo <= 0 unless LEFT).
template <int D, bool MASK, bool LEFT>
__device__ __forceinline__ void dq_half(const lds_char* Ks, const lds_char* Vs, const bf16x8* qf, const bf16x8* df,
                                        f32x16* dq, float c, float lse2, float dlt, int n0, int klo, int khi,
                                        const OperandOffsets<D>& off, int half) {
  using T = DqCfg<D>;
  constexpr int KK = D / 16;
  constexpr int PF = 2;  // K / V operands are fetched PF k-steps ahead of their MFMAs
  f32x16 s = zero16(), dp = zero16();
  uint4 fr[PF + 1][2];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    fr[kk][0] = lds_ld16(Ks + off.row(kk));
    fr[kk][1] = lds_ld16(Vs + off.row(kk));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + PF < KK) {
      fr[(kk + PF) % (PF + 1)][0] = lds_ld16(Ks + off.row(kk + PF));
      fr[(kk + PF) % (PF + 1)][1] = lds_ld16(Vs + off.row(kk + PF));
    }
    __builtin_amdgcn_sched_barrier(0);
    s = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][0]), qf[kk], s);
    dp = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][1]), df[kk], dp);
    __builtin_amdgcn_sched_barrier(0);
  }
  // K^T operands of both k-steps of dQ are read before the exp work
  bf16x8 ka[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) ka[ks][db] = tr_operand<D>(Ks + 16 * ks * T::ROW, off, db);
  }
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
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 sb = to_bf16x8(dsv[8 * ks + 0], dsv[8 * ks + 1], dsv[8 * ks + 2], dsv[8 * ks + 3], dsv[8 * ks + 4],
                                dsv[8 * ks + 5], dsv[8 * ks + 6], dsv[8 * ks + 7]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = mfma32x32x16(ka[ks][db], sb, dq[db]);
  }
}

// BAND: the visible keys of a row form a band (causal and / or a local window).
// LEFT: the band has a left bound (window_left >= 0). Without one, a row's
// visible keys start at key 0, and masked tiles test only their upper bound.
template <int D, bool BAND, bool LEFT>
__global__ __launch_bounds__(256, DqCfg<D>::WAVES_PER_SIMD) void bwd_dq_kernel(BwdParams p) {
  using T = DqCfg<D>;
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

  // key tiles [t_lo, t_hi); the unmasked ones [f_lo, f_hi) lie between masked
  // ones (the band's left edge before, its right edge and the sequence end after)
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

  const uint32_t pitch = (uint32_t)p.Hkv * D * 2;
  const int64_t kvoff = ((int64_t)ck * p.Hkv + g) * D;
  const i32x4 rk = head_rows_rsrc<D>(p.k + kvoff, Lk, pitch);
  const i32x4 rv = head_rows_rsrc<D>(p.v + kvoff, Lk, pitch);
  const uint32_t lds0 = lds_addr(lds);
  if (t_hi > t_lo) issue_kv_dq<D>(lds0 + (t_lo & 1) * T::STAGE, rk, rv, pitch, t_lo * T::BN, wave, lane);

  bf16x8 qf[D / 16], df[D / 16];
  {
    const int64_t off = ((int64_t)(cq + qa) * p.Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = as_bf16x8(qvalid ? ld16(p.q + off + 16 * kk) : zero_u4());
      df[kk] = as_bf16x8(qvalid ? ld16(p.dout + off + 16 * kk) : zero_u4());
    }
  }
  // the row terms of the backward for this lane's query row (the preprocess of
  // the FlashAttention repository guide's Backward Kernels, done here because
  // this workgroup holds the row's dO already): Delta = sum_d dO_d O_d in fp32,
  // lse2 = LSE log2(e), +inf for a row without a visible key so exp2(s - lse2)
  // is exactly 0. Written for the dK / dV kernel, which runs after this one.
  float dlt, lse2;
  {
    const int64_t off = ((int64_t)(cq + qa) * p.Hq + h) * D + 8 * half;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint4 o = qvalid ? ld16(p.out + off + 16 * kk) : zero_u4();
      const uint4 d = __builtin_bit_cast(uint4, df[kk]);
      part += dot8_bf16(d, o);
    }
    dlt = part + __shfl_xor(part, 32);
  }
  const int64_t lidx = (int64_t)h * p.total_q + cq + qa;
  {
    const float l = qvalid ? p.lse[lidx] : -INFINITY;
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  if (qvalid && half == 0) {
    p.delta[lidx] = dlt;
    p.lse2[lidx] = lse2;
  }
  OperandOffsets<D> off;
  operand_offsets<D>(off, lane);

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = zero16();
  const float c = p.scale_log2;

  // masked head, full tiles, masked tail: separate loops so the accumulators
  // keep their registers across iterations
  // one barrier per tile: stage n has landed for every wave, and every wave is
  // done with tile n - 1, whose buffer then takes the copies of tile n + 1
  auto stage_in = [&](int n) {
    wait_vmcnt<0>();
    lds_barrier();
    if (n + 1 < t_hi) issue_kv_dq<D>(lds0 + ((n + 1) & 1) * T::STAGE, rk, rv, pitch, (n + 1) * T::BN, wave, lane);
  };
  auto tile = [&](int n, auto masked) {
    stage_in(n);
    const lds_char* cur = lds + (n & 1) * T::STAGE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      dq_half<D, decltype(masked)::value, LEFT>(cur + kb * 32 * T::ROW, cur + T::TILE + kb * 32 * T::ROW, qf, df, dq, c,
                                          lse2, dlt, n * T::BN + kb * 32, klo, khi, off, half);
  };
  for (int n = t_lo; n < f_lo; ++n) tile(n, std::true_type());
  for (int n = f_lo; n < f_hi; ++n) tile(n, std::false_type());
  for (int n = f_hi; n < t_hi; ++n) tile(n, std::true_type());

  if (qvalid) {
    uint16_t* row = p.dq + ((int64_t)(cq + qi) * p.Hq + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_acc_row(row + db * 32, dq[db], p.scale);
  }
}

// ---------------------------------------------------------------------------
// 3b. query-stationary dQ from the stored dS: dQ = scale * dS K
// ---------------------------------------------------------------------------
// With the stored-dS buffer filled by the dK / dV kernel, the dQ of a query
// block is one product per visible key tile: no S, P or dP to recompute, no
// exponentials. A workgroup owns 128 query rows of one head (32 per wave) and
// walks the visible 64-key tiles in ascending order, staging the K tile and the
// dS^T tile (the 64 keys' rows of the buffer, 128 query columns from the
// block's first row) HBM -> LDS by range-checked DMA, double-buffered; both
// MFMA operands are transposing LDS reads of row-major tiles:
//   dQ^T (32 head-dims x 32 queries) += K^T (head-dims x 16 keys) dS^T (16 keys x queries).
// Tiles that hold hidden pairs (band edges, the sequence's last partial tile)
// mask the dS operand per (query, key): the buffer holds nothing meaningful for
// pairs no dK / dV step visited.

template <int D>
struct DqDsCfg {
  using KV = RowTile<D, 64>;    // K tile: 64 keys
  using DS = RowTile<128, 64>;  // dS^T tile: 64 keys x 128 query columns
  static constexpr int NT = 256;
  static constexpr int BM = 128;  // query rows per workgroup (32 per wave)
  static constexpr int BN = 64;   // keys per tile
  static constexpr int STAGE = KV::BYTES + DS::BYTES;
  static constexpr size_t LDS_BYTES = 2 * STAGE;
  static constexpr int DMA_PER_WAVE = (KV::DMAS + DS::DMAS) / 4;
  static_assert((KV::DMAS + DS::DMAS) % 4 == 0, "copies spread evenly over the 4 waves");
  static_assert(BM == kQueryBlock && BN == key_tile(D), "tile shapes of the host-side plan");
};

template <int D>
__device__ __forceinline__ void issue_k_ds(uint32_t stage, const i32x4& rk, uint32_t pitch_k, const i32x4& rds,
                                           uint32_t pitch_ds, int n0, int wave, int lane) {
  using T = DqDsCfg<D>;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;  // wave-uniform
    if (qd < T::KV::DMAS)
      tile_dma<D, 64>(stage, rk, pitch_k, n0, qd, lane);
    else
      tile_dma<128, 64>(stage + T::KV::BYTES, rds, pitch_ds, n0, qd - T::KV::DMAS, lane);
  }
}

// LDS offsets of the transposing reads of query-column block `blk` (32 columns)
// of a 128-column tile: the tr_operand<128> offsets of head-dim block blk.
__device__ __forceinline__ void tr_block_offsets128(int lane, int blk, uint32_t& t0, uint32_t& t1) {
  constexpr int ROW = 256;
  const int half = lane >> 5;
  const int grp = lane >> 4;
  const int i = lane & 15;
  const int j = i >> 2;
  const int cc = i & 3;
  const int r0 = 8 * half + j;
  const int r1 = r0 + 4;
  const int chunk = blk * 4 + 2 * (grp & 1) + (cc >> 1);
  t0 = r0 * ROW + ((chunk ^ swz<128>(r0)) << 4) + (cc & 1) * 8;
  t1 = r1 * ROW + ((chunk ^ swz<128>(r1)) << 4) + (cc & 1) * 8;
}

// Zero the dS values of keys key0 .. key0 + 7 (one B-operand k-group) that this
// lane's query row does not see: klo <= key < khi (klo only with LEFT).
template <bool LEFT>
__device__ __forceinline__ bf16x8 mask_key_group(const bf16x8& v, int key0, int klo, int khi) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const int k = key0 + 2 * pr;
    const bool a = (!LEFT || k >= klo) && k < khi;
    const bool b = (!LEFT || k + 1 >= klo) && k + 1 < khi;
    w[pr] &= (a ? 0x0000ffffu : 0u) | (b ? 0xffff0000u : 0u);
  }
  return as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
}

// One 64-key tile: 4 k-steps of 16 keys, the operands of k-step s + 1 read
// while k-step s multiplies.
template <int D, bool MASK, bool LEFT>
__device__ __forceinline__ void dq_ds_tile(const lds_char* Ks, const lds_char* Ds, f32x16* dq, int n0, int klo,
                                           int khi, const OperandOffsets<D>& off, uint32_t ds0, uint32_t ds1,
                                           int half) {
  using T = DqDsCfg<D>;
  constexpr int DB = D / 32, NS = T::BN / 16;
  bf16x8 ka[2][DB], sb[2];
  auto load = [&](int s, int slot) {
#pragma unroll
    for (int db = 0; db < DB; ++db) ka[slot][db] = tr_operand<D>(Ks + 16 * s * T::KV::ROW, off, db);
    const uint2 lo = lds_read_tr4(Ds + 16 * s * T::DS::ROW + ds0);
    const uint2 hi = lds_read_tr4(Ds + 16 * s * T::DS::ROW + ds1);
    sb[slot] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };
  load(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + 1 < NS) load(s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 b = MASK ? mask_key_group<LEFT>(sb[s & 1], n0 + 16 * s + 8 * half, klo, khi) : sb[s & 1];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = mfma32x32x16(ka[s & 1][db], b, dq[db]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool BAND, bool LEFT>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_kernel(BwdParams p) {
  using T = DqDsCfg<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  lds_char* lds = (lds_char*)smem;

  const int r = p.Hq / p.Hkv;
  const int64_t L = xcd_logical(blockIdx.x, r);
  const int rank = (int)(L / p.Hq);
  const int h = (int)(L % p.Hq);
  Item item;
  if (!decode_item<false>(p.cu_q, p.cu_k, p.num_seqs, T::BM, p.levels, rank, item)) return;
  const int g = h / r;
  const int mblk = item.m, cq = item.cq, Lq = item.Lq, ck = item.ck, Lk = item.Lk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  // query blocks aligned toward the end of the sequence, as in the forward
  const int q0 = mblk * T::BM - query_lead(Lq, T::BM, T::BN);
  const int qi = q0 + wave * 32 + col;
  const bool qvalid = qi >= 0 && qi < Lq;

  // key tiles [t_lo, t_hi); the unmasked ones [f_lo, f_hi) lie between masked
  // ones (the band's left edge before, its right edge and the sequence end after)
  int t_lo = 0, t_hi = ceil_div(Lk, T::BN), f_lo = 0, f_hi = Lk / T::BN;
  if (BAND) {
    const TileSpan ts = key_tiles(max(q0, 0), min(q0 + T::BM, Lq) - 1, T::BN, Lq, Lk, p.wl, p.wr);
    t_lo = ts.lo;
    t_hi = ts.hi;
    f_lo = ts.full_lo;
    f_hi = max(f_lo, ts.full_hi);
  }
  const int klo = BAND ? band_lo(qi, Lq, Lk, p.wl) : 0;
  const int khi = BAND ? band_hi(qi, Lq, Lk, p.wr) : Lk;

  const uint32_t pitch_k = (uint32_t)p.Hkv * D * 2;
  const i32x4 rk = head_rows_rsrc<D>(p.k + ((int64_t)ck * p.Hkv + g) * D, Lk, pitch_k);
  // dS^T rows of this head and sequence, columns from the block's first query row
  const uint32_t pitch_ds = (uint32_t)p.ds_pitch * 2;
  const i32x4 rds =
      head_rows_rsrc<128>(p.ds + ((int64_t)h * p.total_k + ck) * p.ds_pitch + kDsLead + q0, Lk, pitch_ds);
  const uint32_t lds0 = lds_addr(lds);
  if (t_hi > t_lo) issue_k_ds<D>(lds0 + (t_lo & 1) * T::STAGE, rk, pitch_k, rds, pitch_ds, t_lo * T::BN, wave, lane);

  OperandOffsets<D> off;
  operand_offsets<D>(off, lane);
  uint32_t ds0, ds1;
  tr_block_offsets128(lane, wave, ds0, ds1);

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = zero16();

  // one barrier per tile, as in the dQ kernel
  auto stage_in = [&](int n) {
    wait_vmcnt<0>();
    lds_barrier();
    if (n + 1 < t_hi)
      issue_k_ds<D>(lds0 + ((n + 1) & 1) * T::STAGE, rk, pitch_k, rds, pitch_ds, (n + 1) * T::BN, wave, lane);
  };
  auto tile = [&](int n, auto masked) {
    stage_in(n);
    const lds_char* cur = lds + (n & 1) * T::STAGE;
    dq_ds_tile<D, decltype(masked)::value, LEFT>(cur, cur + T::KV::BYTES, dq, n * T::BN, klo, khi, off, ds0, ds1,
                                                half);
  };
  for (int n = t_lo; n < f_lo; ++n) tile(n, std::true_type());
  for (int n = f_lo; n < f_hi; ++n) tile(n, std::false_type());
  for (int n = f_hi; n < t_hi; ++n) tile(n, std::true_type());

  if (qvalid) {
    uint16_t* row = p.dq + ((int64_t)(cq + qi) * p.Hq + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_acc_row(row + db * 32, dq[db], p.scale);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int D>
static hipError_t launch_prep(const BwdArgs& a, float* delta, float* lse2) {
  const FwdArgs& f = a.f;
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = f.total_q * f.Hq;
  int64_t grid = (rows + RPB - 1) / RPB;
  if (grid > 4096) grid = 4096;
  hipStream_t stream = (hipStream_t)f.stream;
  prof_begin("attn_bwd_prep", stream);
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.dout), static_cast<const uint16_t*>(a.out), a.lse, delta, lse2,
                     (int)f.total_q, f.Hq);
  prof_end(stream);
  return hipGetLastError();
}

template <int D, bool BAND, bool LEFT>
static hipError_t launch_bwd_t(const BwdArgs& a, float* lse2, float* part_dk, float* part_dv, int splits) {
  const FwdArgs& f = a.f;
  hipStream_t stream = (hipStream_t)f.stream;
  BwdParams p;
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
  p.part_dk = nullptr;
  p.part_dv = nullptr;
  p.num_seqs = f.num_seqs;
  p.total_q = (int)f.total_q;
  p.total_k = (int)f.total_k;
  p.Hq = f.Hq;
  p.Hkv = f.Hkv;
  p.splits = 1;
  const Band bd = band_of(f);
  p.wl = bd.wl;
  p.wr = bd.wr;
  p.scale = f.scale;
  p.scale_log2 = f.scale * kLog2e;

  p.ds = static_cast<uint16_t*>(a.ds);
  p.ds_pitch = a.ds_pitch;

  auto run_dkdv = [&](auto store) -> hipError_t {
    using T = DkdvCfg<D>;
    auto kern = bwd_dkdv_kernel<D, BAND, LEFT, decltype(store)::value>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    BwdParams pk = p;
    pk.levels = ceil_div(f.max_k, T::BNK);
    const int64_t grid = grid_for(f.total_k, f.num_seqs, pk.levels, T::BNK, f.Hkv, 1);
    if (grid > 0 && pk.levels > 0) {
      prof_begin("attn_bwd_dkdv", stream);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, pk);
      prof_end(stream);
      e = hipGetLastError();
    }
    return e;
  };
  // the group's query heads split over `splits` items per key block, fp32
  // partial sums, then their ordered reduce (recomputing-dQ path only)
  auto run_dkdv_split = [&]() -> hipError_t {
    using T = DkdvCfg<D>;
    auto kern = bwd_dkdv_kernel<D, BAND, LEFT, false, true>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    BwdParams pk = p;
    pk.levels = ceil_div(f.max_k, T::BNK);
    pk.part_dk = part_dk;
    pk.part_dv = part_dv;
    pk.splits = splits;
    const int64_t grid = grid_for(f.total_k, f.num_seqs, pk.levels, T::BNK, f.Hkv * splits, splits);
    if (grid == 0 || pk.levels == 0) return hipSuccess;
    prof_begin("attn_bwd_dkdv", stream);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, pk);
    prof_end(stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dkdv_reduce(part_dk, part_dv, p.dk, p.dv, f.total_k * f.Hkv * D / 8, splits, f.scale, stream);
  };
  // hw: query heads per workgroup (the recomputing dQ kernel groups a KV
  // group's heads as the forward does; the stored-dS one takes one head)
  auto run_dq = [&](auto kern, size_t lds_bytes, std::atomic<uint64_t>& lds_set, const char* name,
                    int hw) -> hipError_t {
    hipError_t e = lds_limit_once(kern, lds_bytes, lds_set);
    if (e != hipSuccess) return e;
    BwdParams pq = p;
    const int bm = kQueryBlock / hw, hwl = log2_small(hw);
    pq.levels = ceil_div(f.max_q, bm);
    const int64_t grid = grid_for(f.total_q, f.num_seqs, pq.levels, bm, f.Hq >> hwl, (f.Hq / f.Hkv) >> hwl);
    if (grid > 0 && pq.levels > 0) {
      prof_begin(name, stream);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds_bytes, stream, pq);
      prof_end(stream);
      e = hipGetLastError();
    }
    return e;
  };

  if (p.ds) {
    // stored dS (both totals > 0 here): the row terms, then dK / dV, which also
    // writes dS, then dQ = scale * dS K from the stored values
    hipError_t e = launch_prep<D>(a, a.delta, lse2);
    if (e == hipSuccess) e = run_dkdv(std::true_type());
    static std::atomic<uint64_t> lds_set{0};
    if (e == hipSuccess)
      e = run_dq(bwd_dq_ds_kernel<D, BAND, LEFT>, DqDsCfg<D>::LDS_BYTES, lds_set, "attn_bwd_dq_ds", 1);
    return e;
  }
  // recomputing dQ: the dQ kernel first, which also writes the Delta / lse2 rows
  // that dK / dV reads
  if (f.total_q > 0) {
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e =
        run_dq(bwd_dq_kernel<D, BAND, LEFT>, DqCfg<D>::LDS_BYTES, lds_set, "attn_bwd_dq", block_heads(f.Hq / f.Hkv));
    if (e != hipSuccess) return e;
  }
  if (f.total_k > 0) return splits > 1 ? run_dkdv_split() : run_dkdv(std::false_type());
  return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  float* lse2 = reinterpret_cast<float*>(reinterpret_cast<char*>(a.delta) + ws_plane_bytes(a.f.total_q, a.f.Hq));
  // head dims 64 / 128: the dQ kernel forms the row terms itself
  if (D == 256 && a.f.total_q > 0) {
    const hipError_t e = launch_prep<D>(a, a.delta, lse2);
    if (e != hipSuccess) return e;
  }
  // dK / dV query-head splits (the stored-dS path runs without them), as many as
  // the workspace holds
  const int splits =
      a.ds ? 1 : dkdv_splits_within(a.f.total_q, a.f.total_k, a.f.Hq, a.f.Hkv, D, a.ws_bytes);
  char* part = reinterpret_cast<char*>(a.delta) + 2 * ws_plane_bytes(a.f.total_q, a.f.Hq);
  const size_t pb = ws_part_bytes(a.f.total_k, a.f.Hkv, D, splits);
  float* part_dk = splits > 1 ? reinterpret_cast<float*>(part) : nullptr;
  float* part_dv = splits > 1 ? reinterpret_cast<float*>(part + pb) : nullptr;
  if constexpr (D == 256) {
    return launch_bwd_main_d256(a, lse2, part_dk, part_dv, splits);
  } else {
    const Band bd = band_of(a.f);
    if (!bd.band) return launch_bwd_t<D, false, false>(a, lse2, part_dk, part_dv, splits);
    return bd.wl >= 0 ? launch_bwd_t<D, true, true>(a, lse2, part_dk, part_dv, splits)
                      : launch_bwd_t<D, true, false>(a, lse2, part_dk, part_dv, splits);
  }
}

hipError_t launch_bwd(const BwdArgs& a) {
  switch (a.f.D) {
    case 64: return launch_bwd_d<64>(a);
    case 128: return launch_bwd_d<128>(a);
    case 256: return launch_bwd_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// schedule probe: the device decode of ranks, one wave per rank
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void schedule_probe_kernel(const int32_t* cu, int num_seqs, int bm, int levels,
                                                             int count, int32_t* seq_out, int32_t* block_out) {
  const int rank = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rank >= count) return;  // wave-uniform
  int b = -1, m = -1;
  if (!decode_rank(cu, num_seqs, bm, levels, rank, b, m)) {
    b = -1;
    m = -1;
  }
  if ((threadIdx.x & 63) == 0) {
    seq_out[rank] = b;
    block_out[rank] = m;
  }
}

hipError_t launch_schedule_probe(const int32_t* cu_q, int num_seqs, int max_q, int block_m, int32_t* seq_out,
                                 int32_t* block_out, int count, void* stream) {
  const int levels = ceil_div(max_q, block_m);
  const int grid = ceil_div(count, 4);
  hipLaunchKernelGGL(schedule_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, cu_q, num_seqs, block_m,
                     levels, count, seq_out, block_out);
  return hipGetLastError();
}

}  // namespace av
