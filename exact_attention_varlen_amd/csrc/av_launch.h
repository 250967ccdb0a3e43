// av_launch.h — internal interface between the C ABI (av_api.cpp) and the
// kernel launchers. Arguments arrive here already validated.
#ifndef AV_LAUNCH_H
#define AV_LAUNCH_H

#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace av {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs;
  int64_t total_q;
  int64_t total_k;
  int max_q;
  int max_k;
  int Hq;
  int Hkv;
  int D;
  float scale;
  int causal;
  int window_left;   // local window bounds (< 0: unbounded), as passed by the caller
  int window_right;
  void* out;
  float* lse;
  void* stream;
};

// Raise a kernel's dynamic LDS limit on the current device, once per device
// (the attribute belongs to the device's copy of the kernel); `done` holds one
// bit per device ordinal.
template <typename K>
inline hipError_t lds_limit_once(K kern, size_t bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Visible band of a query row i: keys i + (Lk - Lq) - wl .. i + (Lk - Lq) + wr,
// a negative bound meaning unbounded; causal attention caps wr at 0. `band` is
// false for full attention.
struct Band {
  int wl, wr;
  bool band;
};
inline Band band_of(const FwdArgs& a) {
  Band b;
  b.wl = a.window_left < 0 ? -1 : a.window_left;
  b.wr = a.causal ? 0 : (a.window_right < 0 ? -1 : a.window_right);
  b.band = b.wl >= 0 || b.wr >= 0;
  return b;
}

struct BwdArgs {
  FwdArgs f;  // q, k, v, packing, heads, scale, causal, stream (f.out / f.lse unused)
  const void* dout;
  const void* out;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace (Delta, lse2, partial dK / dV): see av_bwd.h
  void* ds;      // stored-dS buffer in the workspace (head dims 64 / 128), or null: dQ recomputes dS
  int ds_pitch;  // its elements per key row
  size_t ws_bytes;  // bytes the workspace holds (bounds the dK / dV split count)
};

// Packing-array check (av_validate.hip): bits of the result word.
constexpr int kSeqlenBadStart = 1;    // cu_seqlens_q[0] or cu_seqlens_k[0] is not 0
constexpr int kSeqlenDecreasing = 2;  // some cu_seqlens entry is smaller than the one before
constexpr int kSeqlenBadTotal = 4;    // cu_seqlens_*[num_seqs] differs from total_q / total_k
constexpr int kSeqlenOverMax = 8;     // some sequence is longer than max_seqlen_q / max_seqlen_k
hipError_t launch_validate_seqlens(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int64_t total_q,
                                   int64_t total_k, int max_q, int max_k, int32_t* result, void* stream);

hipError_t launch_fwd(const FwdArgs& a);

// Split-KV forward (av_fwd_split.hip). The workspace holds the chunks' partial
// outputs, fp32 [splits][total_q][Hq][D], then their log2 row sums, fp32
// [splits][2][Hq][total_q], each part padded to 256 bytes.
constexpr int kMaxSplits = 64;
constexpr int kNumCu = 256;  // compute units of the gfx950 part (8 XCDs x 32)
inline size_t split_pad(size_t b) { return (b + 255) / 256 * 256; }
inline size_t split_part_o_bytes(int64_t total_q, int Hq, int D, int splits) {
  return split_pad((size_t)splits * (size_t)total_q * (size_t)Hq * (size_t)D * sizeof(float));
}
inline size_t split_workspace_bytes(int64_t total_q, int Hq, int D, int splits) {
  if (splits <= 1) return 0;
  return split_part_o_bytes(total_q, Hq, D, splits) +
         split_pad((size_t)splits * 2 * (size_t)Hq * (size_t)total_q * sizeof(float));
}
hipError_t launch_fwd_split(const FwdArgs& a, int splits, void* workspace);
// Persistent forward (av_fwd_persist.hip); sched: kSchedWords zeroed words.
constexpr int kSchedWords = 9;
hipError_t launch_fwd_persistent(const FwdArgs& a, void* sched);
int fwd_num_splits(int num_seqs, int64_t total_q, int max_q, int max_k, int Hq, int Hkv, int D);
hipError_t launch_bwd(const BwdArgs& a);
// The allocation-free backward's device scratch (av_noalloc.hip): its size, and
// its address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_schedule_probe(const int32_t* cu_q, int num_seqs, int max_q, int block_m, int32_t* seq_out,
                                 int32_t* block_out, int count, void* stream);

// per-launch profiling (av_prof.cpp)
void prof_begin(const char* name, hipStream_t stream);
void prof_end(hipStream_t stream);
int prof_enable(int enable);
int prof_count();
int prof_get(int i, char* name, int cap, float* ms);

size_t bwd_workspace_bytes(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D);
// the workspace without dK / dV head splits (the least a backward can run with)
size_t bwd_min_workspace_bytes(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D);
// Workspace of the stored-dS backward (bwd_workspace_bytes plus the dS buffer),
// 0 when that path does not apply; and the dS buffer's row pitch (elements).
size_t bwd_ds_workspace_bytes(int64_t total_q, int64_t total_k, int max_q, int max_k, int Hq, int Hkv, int D);
int bwd_ds_pitch(int max_q);

}  // namespace av

#endif  // AV_LAUNCH_H
