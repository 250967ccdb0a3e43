// av_bwd_d256.hip — backward kernels for head_dim 256: gradients of
// sum(dout * out) for exact varlen GQA attention, deterministic (no atomics,
// every sum in a fixed order). Register-staged variant: Q/dO (resp. K/V) tiles
// go through VGPRs into LDS in row-major and transposed copies.
//
// The FlashAttention repository guide (Backward Kernels) splits the backward
// into a preprocess kernel, a main kernel and a postprocess kernel. Here:
//  1. bwd_delta_kernel   Delta_i = sum_d dO_id * O_id per query row and head
//                        (fp32), written to the caller's workspace.
//  2. bwd_dkdv_kernel    key-stationary: a workgroup owns 128 keys of one KV
//                        head and loops over every query head of that head's
//                        group and every query block that can see the keys,
//                        recomputing P from the LSE:
//                          S = Q K^T, P = exp(S*scale - LSE), dP = dO V^T,
//                          dS = P * (dP - Delta), dV += P^T dO, dK += dS^T Q.
//                        The sum over the group's query heads happens in fp32
//                        registers in a fixed order: no atomics and no scratch.
//  3. bwd_dq_kernel      query-stationary: a workgroup owns 128 query rows of
//                        one head and loops over the visible key tiles in
//                        ascending order: dQ += dS K (fixed order).
// dQ and dK are scaled by softmax_scale at the end.
//
// MFMA lane maps and row permutations are those of av_common.h; the
// transposed operands (Q^T, dO^T for the key-stationary kernel, K^T for the
// query-stationary kernel) are written transposed into LDS at staging time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_common.h"
#include "av_launch.h"

namespace av {

// ---------------------------------------------------------------------------
// staging helpers: 4 consecutive rows x 16 bytes per unit
// ---------------------------------------------------------------------------

struct Rows4V {
  uint4 r[4];
};

__device__ __forceinline__ void rows4_load_v(Rows4V& x, const uint16_t* base, int64_t pitch, int row0, int nvalid,
                                           int col8) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x.r[e] = (row0 + e < nvalid) ? ld16(base + (int64_t)(row0 + e) * pitch + col8) : zero_u4();
}

// rows (row0 .. row0+3) of 8 columns (col8 .. col8+7) -> dst[row][col] row-major
__device__ __forceinline__ void rows4_store_v(const Rows4V& x, uint16_t* dst, int pitch, int row0, int col8) {
#pragma unroll
  for (int e = 0; e < 4; ++e) st16(dst + (row0 + e) * pitch + col8, x.r[e]);
}

// rows (row0 .. row0+3) of 8 columns -> dst[col][row] (transposed), 4 rows per 8-byte write
__device__ __forceinline__ void rows4_store_t_v(const Rows4V& x, uint16_t* dst, int pitch, int row0, int col8) {
  const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&x.r[0]);
  const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&x.r[1]);
  const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&x.r[2]);
  const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&x.r[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint2 lo, hi;
    lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
    lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
    hi.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
    hi.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
    const int c = col8 + 2 * w;
    *reinterpret_cast<uint2*>(dst + c * pitch + row0) = lo;
    *reinterpret_cast<uint2*>(dst + (c + 1) * pitch + row0) = hi;
  }
}

__device__ __forceinline__ float dot8_bf16_v(const uint4& a, const uint4& b) {
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

// ---------------------------------------------------------------------------
// common parameters
// ---------------------------------------------------------------------------

struct BwdParamsV {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int num_seqs;
  int total_q;
  int Hq;
  int Hkv;
  int levels;        // query-block or key-block levels, per kernel
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
};

// LSE in base 2 for a query row; rows outside the sequence or without any
// visible key get +inf so that exp2(s - lse2) is exactly 0 there.
__device__ __forceinline__ float lse_log2_v(const float* lse, int64_t idx, bool valid) {
  if (!valid) return INFINITY;
  const float l = lse[idx];
  return (l == -INFINITY) ? INFINITY : l * kLog2e;
}

// ---------------------------------------------------------------------------
// 2. key-stationary dK / dV
// ---------------------------------------------------------------------------

template <int D>
struct DkdvTileV {
  static constexpr int NT = 256;
  static constexpr int BNK = 128;                  // keys per workgroup (32 per wave)
  static constexpr int BMQ = (D <= 128) ? 64 : 32; // query rows per step
  static constexpr int RP = D + 8;                 // row-major pitch (Q, dO)
  static constexpr int TP = BMQ + 8;               // transposed pitch (Q^T, dO^T)
  static constexpr int UNITS = (BMQ / 4) * (D / 8);  // Rows4V units per tensor per step
  static constexpr int UPT = (UNITS + NT - 1) / NT;  // units per thread per tensor
  static constexpr int OFF_DOS = BMQ * RP;
  static constexpr int OFF_QT = 2 * BMQ * RP;
  static constexpr int OFF_DOT = 2 * BMQ * RP + D * TP;
  static constexpr int OFF_F32 = 2 * BMQ * RP + 2 * D * TP;  // in bf16 elements (even)
  static constexpr size_t LDS_BYTES = (size_t)OFF_F32 * 2 + 2 * BMQ * sizeof(float);
};

template <int D>
struct QdoStageV {
  Rows4V q[DkdvTileV<D>::UPT];
  Rows4V d[DkdvTileV<D>::UPT];
  float lse2;
  float dlt;
};

template <int D>
__device__ __forceinline__ void qdo_load_v(QdoStageV<D>& st, const BwdParamsV& p, int cq, int Lq, int h, int m0) {
  using T = DkdvTileV<D>;
  const int tid = threadIdx.x;
  const int64_t pitch = (int64_t)p.Hq * D;
  const uint16_t* qb = p.q + (int64_t)(cq + m0) * pitch + (int64_t)h * D;
  const uint16_t* db = p.dout + (int64_t)(cq + m0) * pitch + (int64_t)h * D;
  const int nvalid = Lq - m0;
#pragma unroll
  for (int i = 0; i < T::UPT; ++i) {
    const int u = tid + T::NT * i;
    const int rg = u / (D / 8);
    const int c8 = (u % (D / 8)) * 8;
    if (u < T::UNITS) {
      rows4_load_v(st.q[i], qb, pitch, 4 * rg, nvalid, c8);
      rows4_load_v(st.d[i], db, pitch, 4 * rg, nvalid, c8);
    }
  }
  if (tid < T::BMQ) {
    const int i = m0 + tid;
    const bool valid = i < Lq;
    const int64_t idx = (int64_t)h * p.total_q + cq + i;
    st.lse2 = lse_log2_v(p.lse, idx, valid);
    st.dlt = valid ? p.delta[idx] : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void qdo_store_v(const QdoStageV<D>& st, uint16_t* smem) {
  using T = DkdvTileV<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::UPT; ++i) {
    const int u = tid + T::NT * i;
    const int rg = u / (D / 8);
    const int c8 = (u % (D / 8)) * 8;
    if (u < T::UNITS) {
      rows4_store_v(st.q[i], smem, T::RP, 4 * rg, c8);
      rows4_store_v(st.d[i], smem + T::OFF_DOS, T::RP, 4 * rg, c8);
      rows4_store_t_v(st.q[i], smem + T::OFF_QT, T::TP, 4 * rg, c8);
      rows4_store_t_v(st.d[i], smem + T::OFF_DOT, T::TP, 4 * rg, c8);
    }
  }
  float* f = reinterpret_cast<float*>(smem + T::OFF_F32);
  if (tid < T::BMQ) {
    f[tid] = st.lse2;
    f[T::BMQ + tid] = st.dlt;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel_v(BwdParamsV p) {
  using T = DkdvTileV<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  const uint16_t* Qs = smem;
  const uint16_t* dOs = smem + T::OFF_DOS;
  const uint16_t* Qt = smem + T::OFF_QT;
  const uint16_t* dOt = smem + T::OFF_DOT;
  const float* lse2_s = reinterpret_cast<const float*>(smem + T::OFF_F32);
  const float* dlt_s = lse2_s + T::BMQ;

  // work item: (sequence, key block) ranked by descending work, x KV heads
  const int64_t L = xcd_logical(blockIdx.x, 1);
  const int rank = (int)(L / p.Hkv);
  const int g = (int)(L % p.Hkv);
  int b, lvl;
  if (!decode_rank(p.cu_k, p.num_seqs, T::BNK, p.levels, rank, b, lvl)) return;
  const int cq = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - cq;
  const int ck = p.cu_k[b];
  const int Lk = p.cu_k[b + 1] - ck;
  const int nblk = ceil_div(Lk, T::BNK) - 1 - lvl;  // the level counts key blocks from the end
  const int n0 = nblk * T::BNK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int kj = n0 + wave * 32 + col;  // this lane's key (sequence-relative)
  const bool kvalid = kj < Lk;
  const int r = p.Hq / p.Hkv;

  // K^T and V^T operands (B of S = Q K^T and of dP = dO V^T)
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t off = ((int64_t)(ck + kj) * p.Hkv + g) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = as_bf16x8(kvalid ? ld16(p.k + off + 16 * kk) : zero_u4());
      vf[kk] = as_bf16x8(kvalid ? ld16(p.v + off + 16 * kk) : zero_u4());
    }
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  // query blocks that can see a key of this block
  int mfirst = 0;
  if (CAUSAL) {
    mfirst = n0 - (Lk - Lq);
    mfirst = mfirst < 0 ? 0 : (mfirst > Lq ? Lq : mfirst);
  }
  const int sfirst = mfirst / T::BMQ;
  const int nsteps = ceil_div(Lq, T::BMQ) - sfirst;
  const int total = (nsteps > 0) ? nsteps * r : 0;

  const int qrow = kperm(col);
  const int drow = dperm(col);
  const int klim = kj - (Lk - Lq);  // queries i >= klim see this lane's key (causal)

  QdoStageV<D> st;
  if (total > 0) {
    qdo_load_v<D>(st, p, cq, Lq, g * r, sfirst * T::BMQ);
    qdo_store_v<D>(st, smem);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int m0 = (sfirst + it % nsteps) * T::BMQ;
    if (it + 1 < total) {
      const int h1 = g * r + (it + 1) / nsteps;
      const int m1 = (sfirst + (it + 1) % nsteps) * T::BMQ;
      qdo_load_v<D>(st, p, cq, Lq, h1, m1);
    }
    const bool need_mask = CAUSAL && (n0 + T::BNK - 1 - m0 > Lk - Lq);

#pragma unroll
    for (int qb = 0; qb < T::BMQ / 32; ++qb) {
      f32x16 s = zero16(), dp = zero16();
      const uint16_t* qr = Qs + (qb * 32 + qrow) * T::RP + 8 * half;
      const uint16_t* dr = dOs + (qb * 32 + qrow) * T::RP + 8 * half;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32x32x16(as_bf16x8(ld16(qr + 16 * kk)), kf[kk], s);
        dp = mfma32x32x16(as_bf16x8(ld16(dr + 16 * kk)), vf[kk], dp);
      }
      // register v <-> query qb*32 + 16*(v/8) + 8*half + (v%8)
      float l2[16], dl[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qo = qb * 32 + 16 * hh + 8 * half;
        const float4 a0 = *reinterpret_cast<const float4*>(lse2_s + qo);
        const float4 a1 = *reinterpret_cast<const float4*>(lse2_s + qo + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(dlt_s + qo);
        const float4 b1 = *reinterpret_cast<const float4*>(dlt_s + qo + 4);
        l2[8 * hh + 0] = a0.x; l2[8 * hh + 1] = a0.y; l2[8 * hh + 2] = a0.z; l2[8 * hh + 3] = a0.w;
        l2[8 * hh + 4] = a1.x; l2[8 * hh + 5] = a1.y; l2[8 * hh + 6] = a1.z; l2[8 * hh + 7] = a1.w;
        dl[8 * hh + 0] = b0.x; dl[8 * hh + 1] = b0.y; dl[8 * hh + 2] = b0.z; dl[8 * hh + 3] = b0.w;
        dl[8 * hh + 4] = b1.x; dl[8 * hh + 5] = b1.y; dl[8 * hh + 6] = b1.z; dl[8 * hh + 7] = b1.w;
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float pe = fast_exp2(s[v] * p.scale_log2 - l2[v]);
        if (need_mask) {
          const int qi = m0 + qb * 32 + 16 * (v >> 3) + 8 * half + (v & 7);
          pe = (qi >= klim) ? pe : 0.f;
        }
        pv[v] = pe;
        dsv[v] = pe * (dp[v] - dl[v]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pb = to_bf16x8(pv[8 * ks + 0], pv[8 * ks + 1], pv[8 * ks + 2], pv[8 * ks + 3], pv[8 * ks + 4],
                                    pv[8 * ks + 5], pv[8 * ks + 6], pv[8 * ks + 7]);
        const bf16x8 sb = to_bf16x8(dsv[8 * ks + 0], dsv[8 * ks + 1], dsv[8 * ks + 2], dsv[8 * ks + 3],
                                    dsv[8 * ks + 4], dsv[8 * ks + 5], dsv[8 * ks + 6], dsv[8 * ks + 7]);
        const int qo = qb * 32 + 16 * ks + 8 * half;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = db * 32 + drow;
          dv[db] = mfma32x32x16(as_bf16x8(ld16(dOt + d * T::TP + qo)), pb, dv[db]);
          dk[db] = mfma32x32x16(as_bf16x8(ld16(Qt + d * T::TP + qo)), sb, dk[db]);
        }
      }
    }

    __syncthreads();
    if (it + 1 < total) {
      qdo_store_v<D>(st, smem);
      __syncthreads();
    }
  }

  if (kvalid) {
    const int64_t off = ((int64_t)(ck + kj) * p.Hkv + g) * D + 16 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      uint4 a, c, e, f;
      a.x = pack_bf16x2(dk[db][0] * p.scale, dk[db][1] * p.scale);
      a.y = pack_bf16x2(dk[db][2] * p.scale, dk[db][3] * p.scale);
      a.z = pack_bf16x2(dk[db][4] * p.scale, dk[db][5] * p.scale);
      a.w = pack_bf16x2(dk[db][6] * p.scale, dk[db][7] * p.scale);
      c.x = pack_bf16x2(dk[db][8] * p.scale, dk[db][9] * p.scale);
      c.y = pack_bf16x2(dk[db][10] * p.scale, dk[db][11] * p.scale);
      c.z = pack_bf16x2(dk[db][12] * p.scale, dk[db][13] * p.scale);
      c.w = pack_bf16x2(dk[db][14] * p.scale, dk[db][15] * p.scale);
      e.x = pack_bf16x2(dv[db][0], dv[db][1]);
      e.y = pack_bf16x2(dv[db][2], dv[db][3]);
      e.z = pack_bf16x2(dv[db][4], dv[db][5]);
      e.w = pack_bf16x2(dv[db][6], dv[db][7]);
      f.x = pack_bf16x2(dv[db][8], dv[db][9]);
      f.y = pack_bf16x2(dv[db][10], dv[db][11]);
      f.z = pack_bf16x2(dv[db][12], dv[db][13]);
      f.w = pack_bf16x2(dv[db][14], dv[db][15]);
      st16(p.dk + off + db * 32, a);
      st16(p.dk + off + db * 32 + 8, c);
      st16(p.dv + off + db * 32, e);
      st16(p.dv + off + db * 32 + 8, f);
    }
  }
}

// ---------------------------------------------------------------------------
// 3. query-stationary dQ
// ---------------------------------------------------------------------------

template <int D>
struct DqTileV {
  static constexpr int NT = 256;
  static constexpr int BM = 128;   // query rows per workgroup (32 per wave)
  static constexpr int BN = 64;    // keys per tile
  static constexpr int RP = D + 8;
  static constexpr int TP = BN + 8;
  static constexpr int K_UNITS = (BN / 4) * (D / 8);
  static constexpr int K_UPT = (K_UNITS + NT - 1) / NT;
  static constexpr int V_CHUNKS = BN * D / 8 / NT;
  static constexpr int OFF_VS = BN * RP;
  static constexpr int OFF_KT = 2 * BN * RP;
  static constexpr size_t LDS_BYTES = (size_t)(2 * BN * RP + D * TP) * 2;
};

template <int D>
struct KvdStageV {
  Rows4V k[DqTileV<D>::K_UPT];
  uint4 v[DqTileV<D>::V_CHUNKS];
};

template <int D>
__device__ __forceinline__ void kvd_load_v(KvdStageV<D>& st, const uint16_t* kbase, const uint16_t* vbase,
                                         int64_t pitch, int n0, int Lk) {
  using T = DqTileV<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_UPT; ++i) {
    const int u = tid + T::NT * i;
    if (u < T::K_UNITS) rows4_load_v(st.k[i], kbase + (int64_t)n0 * pitch, pitch, 4 * (u / (D / 8)), Lk - n0,
                                   (u % (D / 8)) * 8);
  }
#pragma unroll
  for (int i = 0; i < T::V_CHUNKS; ++i) {
    const int c = tid + T::NT * i;
    const int key = c / (D / 8);
    const int kg = n0 + key;
    st.v[i] = (kg < Lk) ? ld16(vbase + (int64_t)kg * pitch + (c % (D / 8)) * 8) : zero_u4();
  }
}

template <int D>
__device__ __forceinline__ void kvd_store_v(const KvdStageV<D>& st, uint16_t* smem) {
  using T = DqTileV<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_UPT; ++i) {
    const int u = tid + T::NT * i;
    if (u < T::K_UNITS) {
      const int rg = u / (D / 8);
      const int c8 = (u % (D / 8)) * 8;
      rows4_store_v(st.k[i], smem, T::RP, 4 * rg, c8);
      rows4_store_t_v(st.k[i], smem + T::OFF_KT, T::TP, 4 * rg, c8);
    }
  }
#pragma unroll
  for (int i = 0; i < T::V_CHUNKS; ++i) {
    const int c = tid + T::NT * i;
    st16(smem + T::OFF_VS + (c / (D / 8)) * T::RP + (c % (D / 8)) * 8, st.v[i]);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel_v(BwdParamsV p) {
  using T = DqTileV<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  const uint16_t* Ks = smem;
  const uint16_t* Vs = smem + T::OFF_VS;
  const uint16_t* Kt = smem + T::OFF_KT;

  const int r = p.Hq / p.Hkv;
  const int64_t L = xcd_logical(blockIdx.x, r);
  const int rank = (int)(L / p.Hq);
  const int h = (int)(L % p.Hq);
  int b, mblk;
  if (!decode_rank(p.cu_q, p.num_seqs, T::BM, p.levels, rank, b, mblk)) return;
  const int g = h / r;
  const int cq = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - cq;
  const int ck = p.cu_k[b];
  const int Lk = p.cu_k[b + 1] - ck;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q0 = mblk * T::BM;
  const int qi = q0 + wave * 32 + col;
  const bool qvalid = qi < Lq;

  int kend = Lk;
  if (CAUSAL) kend = causal_key_end(min(q0 + T::BM, Lq), Lq, Lk);
  const int ntiles = ceil_div(kend, T::BN);
  const int kfull = CAUSAL ? causal_key_full_end(q0, Lq, Lk) : Lk;

  bf16x8 qf[D / 16], df[D / 16];
  {
    const int64_t off = ((int64_t)(cq + qi) * p.Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = as_bf16x8(qvalid ? ld16(p.q + off + 16 * kk) : zero_u4());
      df[kk] = as_bf16x8(qvalid ? ld16(p.dout + off + 16 * kk) : zero_u4());
    }
  }
  const int64_t lidx = (int64_t)h * p.total_q + cq + qi;
  const float lse2 = lse_log2_v(p.lse, lidx, qvalid);
  const float dlt = qvalid ? p.delta[lidx] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = zero16();

  const int64_t kvpitch = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)ck * kvpitch + (int64_t)g * D;
  const uint16_t* vbase = p.v + (int64_t)ck * kvpitch + (int64_t)g * D;

  KvdStageV<D> st;
  if (ntiles > 0) {
    kvd_load_v<D>(st, kbase, vbase, kvpitch, 0, Lk);
    kvd_store_v<D>(st, smem);
  }
  __syncthreads();

  const int krow = kperm(col);
  const int drow = dperm(col);
  const int qlim = qi + (Lk - Lq);

  for (int n = 0; n < ntiles; ++n) {
    const int n0 = n * T::BN;
    if (n + 1 < ntiles) kvd_load_v<D>(st, kbase, vbase, kvpitch, n0 + T::BN, Lk);
    const bool need_mask = (n0 + T::BN > kfull);

#pragma unroll
    for (int kb = 0; kb < T::BN / 32; ++kb) {
      f32x16 s = zero16(), dp = zero16();
      const uint16_t* kr = Ks + (kb * 32 + krow) * T::RP + 8 * half;
      const uint16_t* vr = Vs + (kb * 32 + krow) * T::RP + 8 * half;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32x32x16(as_bf16x8(ld16(kr + 16 * kk)), qf[kk], s);
        dp = mfma32x32x16(as_bf16x8(ld16(vr + 16 * kk)), df[kk], dp);
      }
      float dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float pe = fast_exp2(s[v] * p.scale_log2 - lse2);
        if (need_mask) {
          const int key = n0 + kb * 32 + 16 * (v >> 3) + 8 * half + (v & 7);
          const bool vis = (key < Lk) && (!CAUSAL || key <= qlim);
          pe = vis ? pe : 0.f;
        }
        dsv[v] = pe * (dp[v] - dlt);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 sb = to_bf16x8(dsv[8 * ks + 0], dsv[8 * ks + 1], dsv[8 * ks + 2], dsv[8 * ks + 3],
                                    dsv[8 * ks + 4], dsv[8 * ks + 5], dsv[8 * ks + 6], dsv[8 * ks + 7]);
        const uint16_t* kt = Kt + drow * T::TP + kb * 32 + 16 * ks + 8 * half;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mfma32x32x16(as_bf16x8(ld16(kt + db * 32 * T::TP)), sb, dq[db]);
      }
    }

    __syncthreads();
    if (n + 1 < ntiles) {
      kvd_store_v<D>(st, smem);
      __syncthreads();
    }
  }

  if (qvalid) {
    uint16_t* row = p.dq + ((int64_t)(cq + qi) * p.Hq + h) * D + 16 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      uint4 a, c;
      a.x = pack_bf16x2(dq[db][0] * p.scale, dq[db][1] * p.scale);
      a.y = pack_bf16x2(dq[db][2] * p.scale, dq[db][3] * p.scale);
      a.z = pack_bf16x2(dq[db][4] * p.scale, dq[db][5] * p.scale);
      a.w = pack_bf16x2(dq[db][6] * p.scale, dq[db][7] * p.scale);
      c.x = pack_bf16x2(dq[db][8] * p.scale, dq[db][9] * p.scale);
      c.y = pack_bf16x2(dq[db][10] * p.scale, dq[db][11] * p.scale);
      c.z = pack_bf16x2(dq[db][12] * p.scale, dq[db][13] * p.scale);
      c.w = pack_bf16x2(dq[db][14] * p.scale, dq[db][15] * p.scale);
      st16(row + db * 32, a);
      st16(row + db * 32 + 8, c);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers (Delta has been computed by the caller)
// ---------------------------------------------------------------------------

template <typename K>
static hipError_t set_lds_limit_v(K kern, size_t bytes, bool& done) {
  if (done) return hipSuccess;
  hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done = true;
  return e;
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_v_t(const BwdArgs& a) {
  const FwdArgs& f = a.f;
  hipStream_t stream = (hipStream_t)f.stream;
  BwdParamsV p;
  p.q = static_cast<const uint16_t*>(f.q);
  p.k = static_cast<const uint16_t*>(f.k);
  p.v = static_cast<const uint16_t*>(f.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.cu_q = f.cu_q;
  p.cu_k = f.cu_k;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.num_seqs = f.num_seqs;
  p.total_q = (int)f.total_q;
  p.Hq = f.Hq;
  p.Hkv = f.Hkv;
  p.scale = f.scale;
  p.scale_log2 = f.scale * kLog2e;
  if (f.total_k > 0) {
    using T = DkdvTileV<D>;
    auto kern = bwd_dkdv_kernel_v<D, CAUSAL>;
    static bool done = false;
    hipError_t e = set_lds_limit_v(kern, T::LDS_BYTES, done);
    if (e != hipSuccess) return e;
    BwdParamsV pk = p;
    pk.levels = ceil_div(f.max_k, T::BNK);
    const int64_t grid = grid_for(f.total_k, f.num_seqs, T::BNK, f.Hkv, 1);
    if (grid > 0 && pk.levels > 0) {
      prof_begin("attn_bwd_dkdv", stream);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, pk);
      prof_end(stream);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (f.total_q > 0) {
    using T = DqTileV<D>;
    auto kern = bwd_dq_kernel_v<D, CAUSAL>;
    static bool done = false;
    hipError_t e = set_lds_limit_v(kern, T::LDS_BYTES, done);
    if (e != hipSuccess) return e;
    BwdParamsV pq = p;
    pq.levels = ceil_div(f.max_q, T::BM);
    const int64_t grid = grid_for(f.total_q, f.num_seqs, T::BM, f.Hq, f.Hq / f.Hkv);
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

hipError_t launch_bwd_main_d256(const BwdArgs& a) {
  return a.f.causal ? launch_bwd_v_t<256, true>(a) : launch_bwd_v_t<256, false>(a);
}

}  // namespace av
