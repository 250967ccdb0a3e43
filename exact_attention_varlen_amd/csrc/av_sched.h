// av_sched.h — work ranking for the varlen kernels (host and device).
//
// A forward work item is (sequence b, query block m, query head h); the key
// blocks an item visits are the non-masked ones only (FlashAttention repository
// guide, Core Abstractions: a block-info helper computes the n-block range for
// causal masking, a seqlen helper tracks varlen offsets, and tile schedulers
// include a varlen-aware one).
//
// Ranking: query blocks are ordered by descending block index m, ties by
// ascending sequence b. Under a causal mask the work of a block grows with m, so
// this runs the longest items first (longest-processing-time order); without a
// mask it runs the long sequences' blocks before the short ones'.
//
//   C(k)  = number of query blocks with index >= k = sum_b max(0, nb_b - k),
//   nb_b  = ceil(Lq_b / block_m).
// Blocks of index k hold ranks [C(k+1), C(k)), in ascending b.
//
// XCD-aware placement: workgroup ids are handed to the 8 XCDs round-robin
// (id % 8). The map below sends the r query heads that share one KV head, for
// the same query block, to consecutive slots of one XCD, so their K/V tiles are
// shared in that XCD's L2, while keeping the global rank order in groups of 8r.
#ifndef AV_SCHED_H
#define AV_SCHED_H

#include <stdint.h>

#define AV_HD __host__ __device__

namespace av {

constexpr int kNumXcd = 8;

AV_HD inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Logical work index of hardware workgroup `hw` (grid a multiple of 8*r).
AV_HD inline int64_t xcd_logical(int64_t hw, int r) {
  const int64_t group = (int64_t)kNumXcd * r;
  const int64_t G = hw / group;
  const int w = (int)(hw - G * group);
  const int xcd = w % kNumXcd;
  const int k = w / kNumXcd;
  return G * group + (int64_t)xcd * r + k;
}

// Grid size of a kernel whose work is (query block rank) x (heads): an upper
// bound on the number of blocks, sum_b ceil(Lq_b / bm) <= total_q / bm + num_seqs,
// times the heads, rounded up to a multiple of 8*r.
AV_HD inline int64_t grid_for(int64_t total_q, int num_seqs, int bm, int heads, int r) {
  const int64_t blocks = total_q / bm + num_seqs;
  const int64_t n = blocks * heads;
  const int64_t group = (int64_t)kNumXcd * r;
  return ((n + group - 1) / group) * group;
}

// Causal block range of a query block: exclusive end of the visible keys of
// the block's last row, clamped to [0, Lk]. Key j is visible to query i when
// j <= i + Lk - Lq.
AV_HD inline int causal_key_end(int q_end, int Lq, int Lk) {
  int e = q_end + (Lk - Lq);
  return e < 0 ? 0 : (e > Lk ? Lk : e);
}

// First key index that may be masked for a query block starting at q0 (the
// keys below it are visible to every row of the block).
AV_HD inline int causal_key_full_end(int q0, int Lq, int Lk) {
  int e = q0 + 1 + (Lk - Lq);
  return e < 0 ? 0 : (e > Lk ? Lk : e);
}

// Host reference of the ranking: enumerate (b, m) in rank order.
inline int64_t rank_enumerate_host(const int32_t* cu, int num_seqs, int bm, int32_t* seq_out,
                                   int32_t* block_out, int64_t capacity) {
  int max_nb = 0;
  for (int b = 0; b < num_seqs; ++b) {
    int nb = ceil_div(cu[b + 1] - cu[b], bm);
    if (nb > max_nb) max_nb = nb;
  }
  int64_t r = 0;
  for (int m = max_nb - 1; m >= 0; --m) {
    for (int b = 0; b < num_seqs; ++b) {
      if (ceil_div(cu[b + 1] - cu[b], bm) > m) {
        if (r < capacity) {
          seq_out[r] = b;
          block_out[r] = m;
        }
        ++r;
      }
    }
  }
  return r;
}

}  // namespace av

#endif  // AV_SCHED_H
