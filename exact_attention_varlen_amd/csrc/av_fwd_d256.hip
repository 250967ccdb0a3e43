// av_fwd_d256.hip — forward kernel for head_dim 256: exact attention over packed
// variable-length sequences with grouped-query heads, bf16 in, fp32
// accumulation, optional LSE. (Register-staged variant: K and V^T go through
// VGPRs into padded LDS tiles; one wave per SIMD.)
//
// What it computes follows the forward loop the FlashAttention repository guide
// describes under Key Patterns (load a Q tile, loop over K/V blocks, online
// softmax with running row max and row sum, store O and LSE) and Core
// Abstractions (online softmax; causal block ranges; varlen offsets). The
// result is the exact softmax(QK^T * scale + mask) V of each packed sequence.
//
// gfx950 design (one workgroup = 4 waves = one query block of 128 rows of one
// query head; each wave owns 32 query rows):
//  * Q^T stays in VGPRs for the whole item as the B operand of S^T = K Q^T.
//  * Per key tile of 64 keys: K is staged row-major and V transposed into LDS
//    (16-byte global loads, prefetched into VGPRs one tile ahead).
//  * S^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16; the key and
//    head-dim row permutations of av_common.h make the fp32 score registers the
//    B operand of the PV product after a bf16 conversion, with no shuffles.
//  * Each lane owns one query column: the running max m, the running sum l and
//    the rescale factor are per-lane values; the row max needs one exchange with
//    lane ^ 32 per tile, and the row sum is only combined at the end.
//  * exp2 with the scale folded in: t = s * (scale * log2 e); the fp32 score is
//    never rounded to bf16 before the exponent.
//  * Masking code runs only on key tiles that cross the causal diagonal or the
//    end of the sequence; tiles past the causal range are never visited.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_common.h"
#include "av_launch.h"

namespace av {

template <int D>
struct FwdTileV {
  static constexpr int BM = 128;     // query rows per workgroup
  static constexpr int BN = 64;      // keys per tile
  static constexpr int NT = 256;     // threads per workgroup
  static constexpr int KP = D + 8;   // LDS row pitch of the K tile (bf16 elements)
  static constexpr int VP = BN + 8;  // LDS row pitch of the V^T tile
  static constexpr int K_CHUNKS = BN * D / 8 / NT;                 // 16-byte K loads per thread
  static constexpr int V_UNITS = (BN / 4) * (D / 8);               // (4 keys x 16 bytes) units per tile
  static constexpr int V_ITERS = (V_UNITS + NT - 1) / NT;          // units per thread
  static constexpr int LDS_ELEMS = BN * KP + D * VP;
  static constexpr size_t LDS_BYTES = (size_t)LDS_ELEMS * 2;
};

struct FwdParamsV {
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
  int levels;  // ceil(max_seqlen_q / BM)
  float scale_log2;  // softmax_scale * log2(e)
};

template <int D>
struct KVStageV {
  uint4 k[FwdTileV<D>::K_CHUNKS];
  uint4 v[FwdTileV<D>::V_ITERS][4];
};

// Global -> VGPR loads of key tile starting at key n0 (sequence-relative).
template <int D>
__device__ __forceinline__ void kv_load_v(KVStageV<D>& st, const uint16_t* kbase, const uint16_t* vbase, int64_t pitch,
                                        int n0, int Lk) {
  using T = FwdTileV<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    const int c = tid + T::NT * i;
    const int key = c / (D / 8);
    const int dc = c % (D / 8);
    const int kg = n0 + key;
    st.k[i] = (kg < Lk) ? ld16(kbase + (int64_t)kg * pitch + dc * 8) : zero_u4();
  }
#pragma unroll
  for (int i = 0; i < T::V_ITERS; ++i) {
    const int u = tid + T::NT * i;
    const int kgrp = u / (D / 8);
    const int dc = u % (D / 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kg = n0 + 4 * kgrp + e;
      st.v[i][e] = (u < T::V_UNITS && kg < Lk) ? ld16(vbase + (int64_t)kg * pitch + dc * 8) : zero_u4();
    }
  }
}

// VGPR -> LDS: K row-major, V transposed (V^T[d][key], 4 keys per 8-byte write).
template <int D>
__device__ __forceinline__ void kv_store_v(const KVStageV<D>& st, uint16_t* Ks, uint16_t* Vt) {
  using T = FwdTileV<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    const int c = tid + T::NT * i;
    const int key = c / (D / 8);
    const int dc = c % (D / 8);
    st16(Ks + key * T::KP + dc * 8, st.k[i]);
  }
#pragma unroll
  for (int i = 0; i < T::V_ITERS; ++i) {
    const int u = tid + T::NT * i;
    if (u < T::V_UNITS) {
      const int kgrp = u / (D / 8);
      const int dc = u % (D / 8);
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&st.v[i][0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&st.v[i][1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&st.v[i][2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&st.v[i][3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // head-dim 2w (low halves) and 2w+1 (high halves) of the 4 keys
        uint2 lo, hi;
        lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
        lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
        hi.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
        hi.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
        const int d = dc * 8 + 2 * w;
        *reinterpret_cast<uint2*>(Vt + d * T::VP + 4 * kgrp) = lo;
        *reinterpret_cast<uint2*>(Vt + (d + 1) * T::VP + 4 * kgrp) = hi;
      }
    }
  }
}

template <int D, bool CAUSAL, bool WRITE_LSE>
__global__ __launch_bounds__(256, 1) void fwd_kernel_v(FwdParamsV p) {
  using T = FwdTileV<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ks = smem;
  uint16_t* Vt = smem + T::BN * T::KP;

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
  const int qi = q0 + wave * 32 + col;  // this lane's query row (sequence-relative)
  const bool qvalid = qi < Lq;

  int kend = Lk;
  if (CAUSAL) kend = causal_key_end(min(q0 + T::BM, Lq), Lq, Lk);
  const int ntiles = ceil_div(kend, T::BN);
  // keys below kfull are visible to every row of the block (and below Lk)
  const int kfull = CAUSAL ? causal_key_full_end(q0, Lq, Lk) : Lk;

  // Q^T operand: 8 consecutive head-dims of this lane's query per k-step.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + ((int64_t)(cq + qi) * p.Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = as_bf16x8(qvalid ? ld16(qrow + 16 * kk) : zero_u4());
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int64_t kvpitch = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)ck * kvpitch + (int64_t)g * D;
  const uint16_t* vbase = p.v + (int64_t)ck * kvpitch + (int64_t)g * D;

  KVStageV<D> st;
  if (ntiles > 0) {
    kv_load_v<D>(st, kbase, vbase, kvpitch, 0, Lk);
    kv_store_v<D>(st, Ks, Vt);
  }
  __syncthreads();

  const int krow = kperm(col);
  const int drow = dperm(col);
  const int qlim = qi + (Lk - Lq);  // last visible key of this lane's query (causal)

  for (int n = 0; n < ntiles; ++n) {
    const int n0 = n * T::BN;
    if (n + 1 < ntiles) kv_load_v<D>(st, kbase, vbase, kvpitch, n0 + T::BN, Lk);

    // S^T = K Q^T for the two 32-key halves of the tile
    f32x16 s[T::BN / 32];
#pragma unroll
    for (int kb = 0; kb < T::BN / 32; ++kb) {
      f32x16 acc = zero16();
      const uint16_t* kr = Ks + (kb * 32 + krow) * T::KP + 8 * half;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) acc = mfma32x32x16(as_bf16x8(ld16(kr + 16 * kk)), qf[kk], acc);
      s[kb] = acc;
    }

    // scale, mask, running max
    const bool need_mask = (n0 + T::BN > kfull);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < T::BN / 32; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float t = s[kb][v] * p.scale_log2;
        if (need_mask) {
          const int key = n0 + kb * 32 + 16 * (v >> 3) + 8 * half + (v & 7);
          const bool vis = (key < Lk) && (!CAUSAL || key <= qlim);
          t = vis ? t : -INFINITY;
        }
        s[kb][v] = t;
        mx = fmaxf(mx, t);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < T::BN / 32; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(s[kb][v] - base);
        s[kb][v] = e;
        lsum += e;
      }
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }

    // O^T += V^T P^T. On masked tiles (the causal diagonal and the sequence
    // tail, where rows with only a few visible keys live and one P value can
    // carry most of a row's weight) P is split into bf16 hi + lo parts so that
    // its rounding does not show in the output.
#pragma unroll
    for (int kb = 0; kb < T::BN / 32; ++kb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[kb][8 * ks + e];
        bf16x8 pb, pl;
        split_bf16x8(pv, pb, pl);
        const uint16_t* vr = Vt + drow * T::VP + kb * 32 + 16 * ks + 8 * half;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 va = as_bf16x8(ld16(vr + db * 32 * T::VP));
          o[db] = mfma32x32x16(va, pb, o[db]);
          if (need_mask) o[db] = mfma32x32x16(va, pl, o[db]);
        }
      }
    }

    __syncthreads();
    if (n + 1 < ntiles) {
      kv_store_v<D>(st, Ks, Vt);
      __syncthreads();
    }
  }

  // epilogue: O = O / l, LSE = ln(2) * (m + log2 l)
  const float l_tot = l_run + xor32(l_run);
  if (qvalid) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.out + ((int64_t)(cq + qi) * p.Hq + h) * D + 16 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      uint4 a, c;
      a.x = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      a.y = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      a.z = pack_bf16x2(o[db][4] * inv, o[db][5] * inv);
      a.w = pack_bf16x2(o[db][6] * inv, o[db][7] * inv);
      c.x = pack_bf16x2(o[db][8] * inv, o[db][9] * inv);
      c.y = pack_bf16x2(o[db][10] * inv, o[db][11] * inv);
      c.z = pack_bf16x2(o[db][12] * inv, o[db][13] * inv);
      c.w = pack_bf16x2(o[db][14] * inv, o[db][15] * inv);
      st16(orow + db * 32, a);
      st16(orow + db * 32 + 8, c);
    }
    if (WRITE_LSE && half == 0) {
      p.lse[(int64_t)h * p.total_q + cq + qi] = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool WRITE_LSE>
static hipError_t launch_fwd_v_t(const FwdArgs& a) {
  using T = FwdTileV<D>;
  auto kern = fwd_kernel_v<D, CAUSAL, WRITE_LSE>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)T::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  FwdParamsV p;
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
  p.levels = ceil_div(a.max_q, T::BM);
  p.scale_log2 = a.scale * kLog2e;
  const int r = a.Hq / a.Hkv;
  const int64_t grid = grid_for(a.total_q, a.num_seqs, T::BM, a.Hq, r);
  if (grid == 0 || p.levels == 0) return hipSuccess;
  hipStream_t stream = (hipStream_t)a.stream;
  prof_begin("attn_fwd", stream);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, p);
  prof_end(stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_v_d(const FwdArgs& a) {
  const bool lse = a.lse != nullptr;
  if (a.causal) return lse ? launch_fwd_v_t<D, true, true>(a) : launch_fwd_v_t<D, true, false>(a);
  return lse ? launch_fwd_v_t<D, false, true>(a) : launch_fwd_v_t<D, false, false>(a);
}

hipError_t launch_fwd_d256(const FwdArgs& a) { return launch_fwd_v_d<256>(a); }

}  // namespace av
