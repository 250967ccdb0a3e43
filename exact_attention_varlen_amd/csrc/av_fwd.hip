// av_fwd.hip — forward kernel: exact attention over packed variable-length
// sequences with grouped-query heads, bf16 in, fp32 accumulation, optional LSE.
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
//  * K and V tiles of 64 keys go HBM -> LDS with buffer_load ... lds (no VGPR
//    staging, out-of-range rows read as zero), double-buffered: the loads of
//    tile n+1 are in flight while tile n is computed. Rows are stored
//    row-major with an XOR swizzle of 16-byte chunks (swz<D>).
//  * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16. V^T comes
//    from the row-major V tile through transposing LDS reads
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
//  * Masking code runs only on key tiles that cross the causal diagonal or the
//    end of the sequence (a separate instantiation of the tile step); tiles
//    past the causal range are never visited. On masked tiles P is split into
//    bf16 hi + lo parts so rows with very few visible keys stay accurate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_common.h"
#include "av_launch.h"
#include "av_tiles.h"

namespace av {

constexpr float kRescaleSlack = 8.0f;

template <int D>
struct FwdTile {
  using KV = RowTile<D, 64>;
  static constexpr int BM = 128;                      // query rows per workgroup
  static constexpr int BN = 64;                       // keys per tile
  static constexpr int NT = 256;                      // threads per workgroup
  static constexpr int ROW = KV::ROW;                 // bytes per key row in LDS
  static constexpr int TILE = KV::BYTES;              // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;              // K then V
  static constexpr size_t LDS_BYTES = 2 * STAGE;      // two stages
  static constexpr int DMA_PER_WAVE = 2 * KV::DMAS / 4;
  static constexpr int WAVES_PER_SIMD = (D <= 128) ? 2 : 1;
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
  int levels;        // ceil(max_seqlen_q / BM)
  float scale_log2;  // |softmax_scale| * log2(e)
  int neg_scale;     // softmax_scale < 0: Q is negated so the scale is positive
};

// Issue this wave's share of the K and V tile copies (keys n0 .. n0+63) into
// the LDS stage at byte address `stage`.
template <int D>
__device__ __forceinline__ void issue_kv(uint32_t stage, const i32x4& rk, const i32x4& rv, uint32_t pitch, int n0,
                                        int wave, int lane) {
  using T = FwdTile<D>;
#pragma unroll
  for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
    const int qd = wave * T::DMA_PER_WAVE + i;  // which 1 KB copy of the stage
    const bool is_v = qd >= T::KV::DMAS;
    tile_dma<D, 64>(stage + (is_v ? T::TILE : 0), is_v ? rv : rk, pitch, n0, is_v ? qd - T::KV::DMAS : qd, lane);
  }
}

// One 64-key tile of the online softmax for one wave (32 query columns):
// S^T = K Q^T for both 32-key halves (two independent MFMA chains, interleaved),
// one running-max update for the tile, then per half P = exp2(S c - m) and
// O^T += V^T P^T. Keeping the rescale decision per tile leaves the exp /
// convert work of one half and the PV products of the other in one basic block.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void fwd_tile(const lds_char* Ks, const lds_char* Vs, const bf16x8* qf, f32x16* o,
                                         float& m_ref, float& l_run, float& l_o, float c, int n0, int Lk, int qlim,
                                         const OperandOffsets<D>& off, int half) {
  using T = FwdTile<D>;
  constexpr int KK = D / 16;
  constexpr int PF = 2;  // K operands are fetched PF k-steps ahead of their MFMAs
  f32x16 s0 = zero16(), s1 = zero16();
  uint4 fr[PF + 1][2];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    fr[kk][0] = lds_ld16(Ks + off.row_off[kk]);
    fr[kk][1] = lds_ld16(Ks + 32 * T::ROW + off.row_off[kk]);
  }
  // fences keep the compiler from sinking each load to just before its MFMA
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + PF < KK) {
      fr[(kk + PF) % (PF + 1)][0] = lds_ld16(Ks + off.row_off[kk + PF]);
      fr[(kk + PF) % (PF + 1)][1] = lds_ld16(Ks + 32 * T::ROW + off.row_off[kk + PF]);
    }
    __builtin_amdgcn_sched_barrier(0);
    s0 = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][0]), qf[kk], s0);
    s1 = mfma32x32x16(as_bf16x8(fr[kk % (PF + 1)][1]), qf[kk], s1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // mask, max over the 64 keys (this lane's 32 and lane ^ 32's 32). Masked
  // scores are excluded by selects, never by -inf arithmetic, so that any
  // finite scale (0 included) is safe.
  uint32_t vis_bits = 0xffffffffu;
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    float x = (v < 16) ? s0[v] : s1[v - 16];
    if (MASK) {
      const int key = n0 + 32 * (v >> 4) + 16 * ((v >> 3) & 1) + 8 * half + (v & 7);
      const bool vis = (key < Lk) && (!CAUSAL || key <= qlim);
      vis_bits = vis ? vis_bits : (vis_bits & ~(1u << v));
      x = vis ? x : -INFINITY;
    }
    mx = fmaxf(mx, x);
  }
  mx = max_xor32(mx);
  const float cand = (mx == -INFINITY) ? -INFINITY : mx * c;
  if (__ballot(cand > m_ref + kRescaleSlack)) {
    const float mn = fmaxf(m_ref, cand);
    // 0 when m_ref = -inf (O and l are still 0); rows that have seen no visible
    // key yet keep mn = -inf and must not form exp2(-inf - -inf)
    const float alpha = fast_exp2(m_ref - (mn == -INFINITY ? 0.f : mn));
    m_ref = mn;
    l_run *= alpha;
    l_o *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
  }
  const float msub = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // V^T operands of this k-step are read before the exp / convert work
      const lds_char* vrow = Vs + (32 * kb + 16 * ks) * T::ROW;
      bf16x8 va[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) va[db] = tr_operand<D>(vrow, off, db);
      __builtin_amdgcn_sched_barrier(0);
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = 16 * kb + 8 * ks + e;
        const float sv = kb ? s1[8 * ks + e] : s0[8 * ks + e];
        float p = fast_exp2(__builtin_fmaf(sv, c, -msub));
        if (MASK) p = ((vis_bits >> v) & 1u) ? p : 0.f;
        pv[e] = p;
        l_run += p;
      }
      bf16x8 pb, pl;
      if (MASK) {
        split_bf16x8(pv, pb, pl);
#pragma unroll
        for (int e = 0; e < 8; ++e) l_o += pv[e];
      } else {
        uint4 u;
        u.x = pack_bf16x2(pv[0], pv[1]);
        u.y = pack_bf16x2(pv[2], pv[3]);
        u.z = pack_bf16x2(pv[4], pv[5]);
        u.w = pack_bf16x2(pv[6], pv[7]);
        l_o = add_bf16x2(u.x, l_o);
        l_o = add_bf16x2(u.y, l_o);
        l_o = add_bf16x2(u.z, l_o);
        l_o = add_bf16x2(u.w, l_o);
        pb = as_bf16x8(u);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        o[db] = mfma32x32x16(va[db], pb, o[db]);
        if (MASK) o[db] = mfma32x32x16(va[db], pl, o[db]);
      }
    }
  }
}

template <int D, bool CAUSAL, bool WRITE_LSE>
__global__ __launch_bounds__(256, FwdTile<D>::WAVES_PER_SIMD) void fwd_kernel(FwdParams p) {
  using T = FwdTile<D>;
  extern __shared__ __align__(16) uint16_t smem[];
  lds_char* lds = (lds_char*)smem;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q0 = mblk * T::BM;
  const int qi = q0 + wave * 32 + col;  // this lane's query row (sequence-relative)
  const bool qvalid = qi < Lq;

  int kend = Lk;
  if (CAUSAL) kend = causal_key_end(min(q0 + T::BM, Lq), Lq, Lk);
  const int ntiles = ceil_div(kend, T::BN);
  // tiles [0, nfull) need no mask: every key is below Lk and visible to every row
  const int kfull = CAUSAL ? causal_key_full_end(q0, Lq, Lk) : Lk;
  const int nfull = min(ntiles, kfull / T::BN);

  // K / V buffer resources for this (sequence, KV head): rows past Lk read as 0
  const uint32_t pitch = (uint32_t)p.Hkv * D * 2;
  const int64_t kvoff = ((int64_t)ck * p.Hkv + g) * D;
  const i32x4 rk = head_rows_rsrc<D>(p.k + kvoff, Lk, pitch);
  const i32x4 rv = head_rows_rsrc<D>(p.v + kvoff, Lk, pitch);
  const uint32_t lds0 = lds_addr(lds);

  if (ntiles > 0) issue_kv<D>(lds0, rk, rv, pitch, 0, wave, lane);

  // Q^T operand: 8 consecutive head-dims of this lane's query per k-step
  // (sign-flipped when the scale is negative, so the scale applied is positive).
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + ((int64_t)(cq + qi) * p.Hq + h) * D + 8 * half;
    const uint32_t flip = p.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 u = qvalid ? ld16(qrow + 16 * kk) : zero_u4();
      u.x ^= flip;
      u.y ^= flip;
      u.z ^= flip;
      u.w ^= flip;
      qf[kk] = as_bf16x8(u);
    }
  }

  // per-lane LDS byte offsets of the MFMA operand reads
  OperandOffsets<D> off;
  operand_offsets<D>(off, lane);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  float m_ref = -INFINITY;
  float l_run = 0.f;  // sum of P (fp32): the LSE
  float l_o = 0.f;    // sum of the P values as they enter the PV product: normalises O
  const float c = p.scale_log2;
  const int qlim = qi + (Lk - Lq);  // last visible key of this lane's query (causal)

  // Full tiles first, then the masked ones (causal diagonal, sequence tail), as
  // two loops so that the accumulators keep their registers across iterations.
  auto stage_in = [&](int n) {
    if (n + 1 < ntiles) {
      issue_kv<D>(lds0 + ((n + 1) & 1) * T::STAGE, rk, rv, pitch, (n + 1) * T::BN, wave, lane);
      wait_vmcnt<T::DMA_PER_WAVE>();  // this wave's copies of tile n have landed
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();  // ... and every other wave's
  };
  for (int n = 0; n < nfull; ++n) {
    stage_in(n);
    const lds_char* cur = lds + (n & 1) * T::STAGE;
    fwd_tile<D, false, CAUSAL>(cur, cur + T::TILE, qf, o, m_ref, l_run, l_o, c, n * T::BN, Lk, qlim, off, half);
    lds_barrier();  // stage (n & 1) is free for tile n + 2
  }
  for (int n = nfull; n < ntiles; ++n) {
    stage_in(n);
    const lds_char* cur = lds + (n & 1) * T::STAGE;
    fwd_tile<D, true, CAUSAL>(cur, cur + T::TILE, qf, o, m_ref, l_run, l_o, c, n * T::BN, Lk, qlim, off, half);
    lds_barrier();
  }

  // epilogue: O = O / l, LSE = ln(2) * (m + log2 l)
  const float l_tot = add_xor32(l_run);
  const float lo_tot = add_xor32(l_o);
  if (qvalid) {
    const float inv = (lo_tot > 0.f) ? 1.f / lo_tot : 0.f;
    uint16_t* orow = p.out + ((int64_t)(cq + qi) * p.Hq + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_acc_row(orow + db * 32, o[db], inv);
    if (WRITE_LSE && half == 0) {
      p.lse[(int64_t)h * p.total_q + cq + qi] =
          (l_tot > 0.f && m_ref != -INFINITY) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool WRITE_LSE>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using T = FwdTile<D>;
  auto kern = fwd_kernel<D, CAUSAL, WRITE_LSE>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)T::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
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
  p.levels = ceil_div(a.max_q, T::BM);
  p.scale_log2 = fabsf(a.scale) * kLog2e;
  p.neg_scale = a.scale < 0.f ? 1 : 0;
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
static hipError_t launch_fwd_d(const FwdArgs& a) {
  const bool lse = a.lse != nullptr;
  if (a.causal) return lse ? launch_fwd_t<D, true, true>(a) : launch_fwd_t<D, true, false>(a);
  return lse ? launch_fwd_t<D, false, true>(a) : launch_fwd_t<D, false, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.D) {
    case 64: return launch_fwd_d<64>(a);
    case 128: return launch_fwd_d<128>(a);
    case 256: return launch_fwd_d256(a);
    default: return hipErrorInvalidValue;
  }
}

int64_t fwd_grid_size(int64_t total_q, int num_seqs, int Hq, int Hkv) {
  return grid_for(total_q, num_seqs, 128, Hq, Hq / Hkv);
}

}  // namespace av
