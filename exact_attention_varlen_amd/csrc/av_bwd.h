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
  uint16_t* ds;      // stored dS^T, bf16 [Hq][total_k][ds_pitch] (head dims 64 / 128), or null
  int ds_pitch;      // elements per key row of ds: kDsLead + max_seqlen_q rounded up to 128
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

// Query-head splits of the dK / dV work (head_dim 256 and, with few work items,
// 64 / 128). The kernels are key-stationary: a work item is a key block of one KV
// head and sums the group's r query heads in registers. With few key blocks x KV
// heads (short sequences, few KV heads) that leaves most compute units idle, so
// the group's heads are split over s items, each writing fp32 partial sums that
// bwd_dkdv_reduce_kernel adds in split order (deterministic, no atomics).
// head_dim 256 (one workgroup per CU, long items): the smallest divisor s of r
// with (key blocks x KV heads x s) >= 2048 work items (8 per compute unit, so
// longest-first ordering can balance causal work), else r. head_dim 64 / 128:
// no split while there are at least 256 items (one per compute unit); below
// that the smallest divisor s of r giving >= 1024 items, else r.
// Key blocks are counted as total_k / 128, a lower bound of sum_b ceil(Lk_b / 128).
inline int dkdv_splits(int64_t total_k, int Hq, int Hkv, int D) {
  if (Hkv <= 0) return 1;
  const int r = Hq / Hkv;
  const int64_t base = (total_k / 128 > 0 ? total_k / 128 : 1) * (int64_t)Hkv;
  if (D != 256 && base >= 256) return 1;
  const int64_t want = D == 256 ? 2048 : 1024;
  for (int s = 1; s <= r; ++s) {
    if (r % s == 0 && base * s >= want) return s;
  }
  return r > 0 ? r : 1;
}

// Stored dS (head dims 64 / 128): the dK / dV kernel writes dS = P (dP - Delta)
// in bf16 as it forms it, and the dQ kernel then only multiplies it by K instead
// of recomputing S, P, dP and dS. Layout: one row per (query head, key),
// [Hq][total_k][ds_pitch], query rows of the key's sequence along the row,
// starting at column kDsLead (the dQ kernel's query blocks, aligned toward the
// sequence end, start up to 64 rows before row 0). Entries of (query, key)
// pairs that no dK / dV step visits are never written; the dQ kernel masks every
// pair it does not know to be visible.
constexpr int kDsLead = 64;
inline int ds_pitch_of(int max_q) { return kDsLead + (max_q + 127) / 128 * 128; }
// Bytes of the dS buffer, or 0 when this path does not apply: head dim 256, an
// empty problem, or one key sequence's rows spanning 2 GiB or more of the buffer
// (32-bit offsets within a sequence).
inline size_t ds_buffer_bytes(int64_t total_q, int64_t total_k, int max_q, int max_k, int Hq, int D) {
  if (D > 128 || total_q <= 0 || total_k <= 0 || max_q <= 0 || max_k <= 0) return 0;
  const int64_t pitch_bytes = 2 * (int64_t)ds_pitch_of(max_q);
  if ((int64_t)(max_k + 64) * pitch_bytes >= ((int64_t)1 << 31)) return 0;
  return ws_pad((size_t)Hq * (size_t)total_k * (size_t)pitch_bytes);
}

inline size_t ws_part_bytes(int64_t total_k, int Hkv, int D, int splits) {
  return splits > 1 ? ws_pad((size_t)splits * (size_t)total_k * (size_t)Hkv * (size_t)D * sizeof(float)) : 0;
}

// Backward workspace: Delta and lse2 planes, then the partial dK / dV sums.
inline size_t bwd_ws_bytes_for(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D, int splits) {
  return 2 * ws_plane_bytes(total_q, Hq) + 2 * ws_part_bytes(total_k, Hkv, D, splits);
}

// The split count a backward runs with: dkdv_splits, lowered to the largest
// divisor of r whose workspace fits in `limit` bytes (the allocation-free entry
// point's fixed scratch); 1 always fits where the call was accepted.
inline int dkdv_splits_within(int64_t total_q, int64_t total_k, int Hq, int Hkv, int D, size_t limit) {
  const int want = dkdv_splits(total_k, Hq, Hkv, D);
  const int r = Hkv > 0 ? Hq / Hkv : 1;
  for (int s = want; s > 1; --s) {
    if (r % s == 0 && bwd_ws_bytes_for(total_q, total_k, Hq, Hkv, D, s) <= limit) return s;
  }
  return 1;
}

}  // namespace av

#endif  // AV_BWD_H
