// av_fwd.hip — launch of the forward kernel (av_fwd_kernel.h) with one
// workgroup per (query block, query head) visiting every visible key tile.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "av_fwd_kernel.h"

namespace av {

template <int D, int MODE, bool WRITE_LSE>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  constexpr int BM = FwdBlock<D>::BM, BN = FwdBlock<D>::BN;
  using T = FwdCfg<D, BM, BN>;
  auto kern = fwd_kernel<D, BM, BN, MODE, WRITE_LSE>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once(kern, T::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
  }
  FwdParams p = fwd_params(a, T::BM);
  const int r = a.Hq / a.Hkv;
  const int64_t grid = grid_for(a.total_q, a.num_seqs, p.levels, p.bm, a.Hq >> p.hw_log2, r >> p.hw_log2);
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
  const Band bd = band_of(a);
  if (bd.wl >= 0) return lse ? launch_fwd_t<D, 2, true>(a) : launch_fwd_t<D, 2, false>(a);
  if (bd.band) return lse ? launch_fwd_t<D, 1, true>(a) : launch_fwd_t<D, 1, false>(a);
  return lse ? launch_fwd_t<D, 0, true>(a) : launch_fwd_t<D, 0, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.D) {
    case 64: return launch_fwd_d<64>(a);
    case 128: return launch_fwd_d<128>(a);
    case 256: return launch_fwd_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace av
