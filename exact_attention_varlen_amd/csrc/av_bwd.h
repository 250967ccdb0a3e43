// av_bwd.h — definitions shared by the backward kernels (av_bwd.hip for head
// dims 64 / 128, av_bwd_d256.hip for head dim 256).
#ifndef AV_BWD_H
#define AV_BWD_H

#include <stddef.h>
#include <stdint.h>

#include "av_common.h"

namespace av {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  float* delta;       // Delta = rowsum(dO * O) [Hq][total_q] (written by the dQ kernel at head dims 64 / 128)
  float* lse2;        // LSE * log2(e), +inf for rows without a visible key (likewise)
  const uint16_t* out;  // forward output O and its LSE (read by the dQ kernel at head dims 64 / 128)
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* part_dk;    // fp32 partial dK / dV per head split (head dim 256 with splits > 1)
  float* part_dv;
  int num_seqs;
  int total_q;
  int total_k;
  int Hq;
  int Hkv;
  int splits;        // query-head splits of the dK / dV work (1: write dK / dV directly)
  int levels;        // query-block or key-block levels, per kernel
  int wl, wr;        // visible band of a row (keys i + Lk - Lq - wl .. + wr; < 0: unbounded)
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
};

// Copy of 64 consecutive fp32 row values (rows row0 .. row0 + 63 of one head's
// plane) into LDS at `dst`; rows past the sequence read as 0.
__device__ __forceinline__ void rows64_f32_dma(uint32_t dst, const i32x4& rsrc, int row0, int lane) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(dst), "v"((uint32_t)(row0 + lane) * 4u), "s"(rsrc)
      : "memory", "m0");
}

// Workspace layout: Delta [Hq][total_q] fp32, lse2 [Hq][total_q] fp32, then,
// when the dK / dV work of head dim 256 is split over query heads, the fp32
// partial sums [splits][total_k][Hkv][D] of dK and then of dV. Each part is
// padded to 256 bytes.
inline size_t ws_pad(size_t b) { return (b + 255) / 256 * 256; }
inline size_t ws_plane_bytes(int64_t total_q, int Hq) { return ws_pad((size_t)total_q * (size_t)Hq * sizeof(float)); }

// Query-head splits of the head dim 256 dK / dV work: the smallest divisor s of
// the group size r with (key blocks x KV heads x s) >= 2048 work items (8 per
// compute unit, so longest-first ordering can balance causal work), else r.
// Key blocks are counted as total_k / 128, a lower bound of sum_b ceil(Lk_b / 128).
inline int dkdv_splits(int64_t total_k, int Hq, int Hkv, int D) {
  if (D != 256 || Hkv <= 0) return 1;
  const int r = Hq / Hkv;
  const int64_t base = (total_k / 128 > 0 ? total_k / 128 : 1) * (int64_t)Hkv;
  for (int s = 1; s <= r; ++s) {
    if (r % s == 0 && base * s >= 2048) return s;
  }
  return r > 0 ? r : 1;
}

inline size_t ws_part_bytes(int64_t total_k, int Hkv, int D, int splits) {
  return splits > 1 ? ws_pad((size_t)splits * (size_t)total_k * (size_t)Hkv * (size_t)D * sizeof(float)) : 0;
}

}  // namespace av

#endif  // AV_BWD_H
