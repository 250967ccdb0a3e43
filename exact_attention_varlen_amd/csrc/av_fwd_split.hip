// av_fwd_split.hip — split-KV forward: the key tiles of each work item are
// cut into contiguous chunks that run as separate workgroups, each writing a
// partial (O, row sums) for its keys, and a combine kernel merges them
// (FlashAttention repository guide, Public API: num_splits; Forward Kernels:
// the split-KV combine of partial outputs and their LSEs).
//
// Merge identity: if chunk s holds P_s = sum_{j in s} 2^(t_j - m) with its own
// normalised output O_s = sum_{j in s} 2^(t_j - m) v_j / P_s, then over all
// keys O = sum_s P_s O_s / sum_s P_s and log2 P = log2 sum_s P_s. Each chunk
// reports log2 P_s with its own reference m_s, so the combine rescales by
// 2^(log2 P_s - max_s log2 P_s). Two such sums are kept per chunk, as in the
// one-pass kernel: the fp32 sum of P for the LSE, and the sum of the bf16 P
// that entered the PV product for O's weights, so O keeps the one-pass
// kernel's cancellation of P's rounding.
//
// Use: shapes with too few (query block, head) items to fill the chip, e.g.
// short query chunks against long key sequences.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "av_fwd_kernel.h"

namespace av {

// One group of D / 4 lanes per (token, query head) pair, 4 head-dims per lane.
template <int D>
struct CombineCfg {
  static constexpr int NT = 256;
  static constexpr int LANES = D / 4;           // lanes per pair
  static constexpr int PAIRS = NT / LANES;      // pairs per workgroup
};

template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_l,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse,
                                                          int total_q, int Hq, int splits) {
  using C = CombineCfg<D>;
  const int64_t npairs = (int64_t)total_q * Hq;
  const int64_t pair = (int64_t)blockIdx.x * C::PAIRS + threadIdx.x / C::LANES;
  if (pair >= npairs) return;
  const int li = threadIdx.x % C::LANES;
  const int row = (int)(pair / Hq);
  const int h = (int)(pair % Hq);
  const int64_t plane = npairs;  // Hq * total_q
  const float* lrow = part_l + (int64_t)h * total_q + row;

  // reference points: the largest log2 sums over the chunks
  float mr = -INFINITY, mo = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    mr = fmaxf(mr, lrow[(int64_t)s * 2 * plane]);
    mo = fmaxf(mo, lrow[(int64_t)s * 2 * plane + plane]);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f, rsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float lr = lrow[(int64_t)s * 2 * plane];
    const float lo = lrow[(int64_t)s * 2 * plane + plane];
    if (lr != -INFINITY) rsum += exp2f(lr - mr);
    if (lo != -INFINITY) {  // chunks without a visible key wrote no O
      const float w = exp2f(lo - mo);
      const float4 o = *reinterpret_cast<const float4*>(part_o + ((int64_t)s * npairs + pair) * D + 4 * li);
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
      wsum += w;
    }
  }
  const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
  uint2 wv;
  wv.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  wv.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(out + pair * D + 4 * li) = wv;
  if (lse != nullptr && li == 0)
    lse[(int64_t)h * total_q + row] = (mr == -INFINITY) ? -INFINITY : (mr + log2f(rsum)) * kLn2;
}

template <int D, int MODE>
static hipError_t launch_split_t(const FwdArgs& a, int splits, float* part_o, float* part_l) {
  constexpr int BM = FwdBlock<D>::BM, BN = FwdBlock<D>::BN;
  using T = FwdCfg<D, BM, BN>;
  auto kern = fwd_kernel<D, BM, BN, MODE, false, true>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
  }
  FwdParams p = fwd_params(a, T::BM);
  p.part_o = part_o;
  p.part_l = part_l;
  p.splits = splits;
  const int r = a.Hq / a.Hkv;
  const int64_t grid = grid_for(a.total_q, a.num_seqs, p.levels, p.bm, (a.Hq >> p.hw_log2) * splits, r >> p.hw_log2);
  if (grid == 0 || p.levels == 0) return hipSuccess;
  hipStream_t stream = (hipStream_t)a.stream;
  prof_begin("attn_fwd_split", stream);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), T::LDS_BYTES, stream, p);
  prof_end(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  using C = CombineCfg<D>;
  const int64_t cgrid = ((int64_t)a.total_q * a.Hq + C::PAIRS - 1) / C::PAIRS;
  prof_begin("attn_fwd_combine", stream);
  hipLaunchKernelGGL(fwd_combine_kernel<D>, dim3((unsigned)cgrid), dim3(C::NT), 0, stream, part_o, part_l,
                     static_cast<uint16_t*>(a.out), a.lse, (int)a.total_q, a.Hq, splits);
  prof_end(stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_split_d(const FwdArgs& a, int splits, float* part_o, float* part_l) {
  const Band bd = band_of(a);
  if (bd.wl >= 0) return launch_split_t<D, 2>(a, splits, part_o, part_l);
  if (bd.band) return launch_split_t<D, 1>(a, splits, part_o, part_l);
  return launch_split_t<D, 0>(a, splits, part_o, part_l);
}

hipError_t launch_fwd_split(const FwdArgs& a, int splits, void* workspace) {
  if (splits <= 1) return launch_fwd(a);
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_l = reinterpret_cast<float*>(ws + split_part_o_bytes(a.total_q, a.Hq, a.D, splits));
  switch (a.D) {
    case 64: return launch_split_d<64>(a, splits, part_o, part_l);
    case 128: return launch_split_d<128>(a, splits, part_o, part_l);
    case 256: return launch_split_d<256>(a, splits, part_o, part_l);
    default: return hipErrorInvalidValue;
  }
}

// Work items of the one-pass grid (an upper bound from the sizes the host
// knows) against the workgroups the chip holds at once; the chosen count is
// the smallest whose last wave of workgroups is at least 90 % as full as the
// best count's, with every chunk at least 4 key tiles long.
int fwd_num_splits(int num_seqs, int64_t total_q, int max_q, int max_k, int Hq, int Hkv, int D) {
  (void)Hkv;
  const int bm = 128;
  const int bn = (D <= 128) ? 64 : 32;
  const int64_t slots = (int64_t)kNumCu * ((D <= 128) ? 2 : 1);
  const int64_t blocks_a = total_q / bm + num_seqs;
  const int64_t blocks_b = (int64_t)num_seqs * ((max_q + bm - 1) / bm);
  const int64_t items = (blocks_a < blocks_b ? blocks_a : blocks_b) * Hq;
  if (items <= 0) return 1;
  const int tiles = (max_k + bn - 1) / bn;
  int smax = tiles / 4;
  if (smax > kMaxSplits) smax = kMaxSplits;
  if (smax <= 1) return 1;
  auto eff = [&](int s) {
    const int64_t n = items * s;
    const int64_t waves = (n + slots - 1) / slots;
    return (double)n / (double)(waves * slots);
  };
  double best = 0.0;
  for (int s = 1; s <= smax; ++s) best = eff(s) > best ? eff(s) : best;
  for (int s = 1; s <= smax; ++s)
    if (eff(s) >= 0.9 * best) return s;
  return 1;
}

}  // namespace av
