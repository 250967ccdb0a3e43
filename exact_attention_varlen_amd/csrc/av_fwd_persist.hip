// av_fwd_persist.hip — launch of the forward kernel with persistent, varlen-
// aware scheduling (fwd_kernel_persistent in av_fwd_kernel.h): one workgroup
// per concurrent slot of the chip, work items taken from per-XCD queues.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "av_fwd_kernel.h"

namespace av {

template <int D, int MODE, bool WRITE_LSE>
static hipError_t launch_persist_t(const FwdArgs& a, unsigned int* sched) {
  constexpr int BM = FwdBlock<D>::BM, BN = FwdBlock<D>::BN;
  using T = FwdCfg<D, BM, BN>;
  auto kern = fwd_kernel_persistent<D, BM, BN, MODE, WRITE_LSE>;
  constexpr size_t lds = T::LDS_BYTES + 16;  // K / V buffers, then two item slots and a queue cursor
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once(kern, lds, lds_set);
    if (e != hipSuccess) return e;
  }
  FwdParams p = fwd_params(a, T::BM);
  p.sched = sched;
  const int r = a.Hq / a.Hkv;
  const int64_t n_items = grid_for(a.total_q, a.num_seqs, p.levels, p.bm, a.Hq >> p.hw_log2, r >> p.hw_log2);
  if (n_items == 0 || p.levels == 0) return hipSuccess;
  const int64_t slots = (int64_t)kNumCu * T::MIN_BLOCKS_PER_CU;
  const int64_t grid = n_items < slots ? n_items : slots;
  hipStream_t stream = (hipStream_t)a.stream;
  prof_begin("attn_fwd_persistent", stream);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(T::NT), lds, stream, p, (unsigned int)n_items);
  prof_end(stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_persist_d(const FwdArgs& a, unsigned int* sched) {
  const bool lse = a.lse != nullptr;
  const Band bd = band_of(a);
  if (bd.wl >= 0) return lse ? launch_persist_t<D, 2, true>(a, sched) : launch_persist_t<D, 2, false>(a, sched);
  if (bd.band) return lse ? launch_persist_t<D, 1, true>(a, sched) : launch_persist_t<D, 1, false>(a, sched);
  return lse ? launch_persist_t<D, 0, true>(a, sched) : launch_persist_t<D, 0, false>(a, sched);
}

hipError_t launch_fwd_persistent(const FwdArgs& a, void* sched) {
  unsigned int* s = static_cast<unsigned int*>(sched);
  switch (a.D) {
    case 64: return launch_persist_d<64>(a, s);
    case 128: return launch_persist_d<128>(a, s);
    case 256: return launch_persist_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace av
