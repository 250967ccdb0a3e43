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
// bound on the number of blocks, sum_b ceil(Lq_b / bm), times the heads, rounded
// up to a multiple of 8*r. Two bounds hold, the smaller is taken:
// total_q / bm + num_seqs (a partial block per sequence at most) and
// num_seqs * levels, levels = ceil(max_seqlen / bm) (the first is tight for a few
// long sequences, the second for many short ones). Workgroups past the last
// block find no work, but each still decodes its rank first.
AV_HD inline int64_t grid_for(int64_t total_q, int num_seqs, int levels, int bm, int heads, int r) {
  const int64_t by_tokens = total_q / bm + num_seqs;
  const int64_t by_lengths = (int64_t)num_seqs * levels;
  const int64_t blocks = by_tokens < by_lengths ? by_tokens : by_lengths;
  const int64_t n = blocks * heads;
  const int64_t group = (int64_t)kNumXcd * r;
  return ((n + group - 1) / group) * group;
}

// Rows by which the first query block of a sequence starts before row 0: the
// padding of ceil(Lq / bm) blocks of bm rows, rounded down to whole key tiles
// of bn rows. Blocks start at mblk bm - lead; there are still ceil(Lq / bm) of
// them, and the last one overhangs the sequence by less than bn rows.
AV_HD inline int query_lead(int Lq, int bm, int bn) {
  const int pad = (Lq + bm - 1) / bm * bm - Lq;
  return pad / bn * bn;
}

// Visible keys of a query row, as a band around the bottom-right-aligned
// diagonal (FlashAttention repository guide, Public API: causal,
// window_size_left / window_size_right). Key j is visible to query i when
//   i + (Lk - Lq) - wl <= j <= i + (Lk - Lq) + wr,
// a negative bound meaning none on that side; causal attention is wr = 0.
// band_lo / band_hi are the row's first visible key and one past its last,
// clamped to [0, Lk] (band_lo >= band_hi: no visible key).
AV_HD inline int clamp_key(int64_t e, int Lk) { return e < 0 ? 0 : (e > Lk ? Lk : (int)e); }
AV_HD inline int band_lo(int i, int Lq, int Lk, int wl) {
  return wl < 0 ? 0 : clamp_key((int64_t)i + (Lk - Lq) - wl, Lk);
}
AV_HD inline int band_hi(int i, int Lq, int Lk, int wr) {
  return wr < 0 ? Lk : clamp_key((int64_t)i + (Lk - Lq) + wr + 1, Lk);
}

// Key range of a block of query rows [r0, r1] (inclusive, r1 < Lq): the keys
// some row sees, [lo, hi), and the keys every row sees, [full_lo, full_hi)
// (empty when full_lo >= full_hi).
struct KeyRange {
  int lo, hi, full_lo, full_hi;
};
AV_HD inline KeyRange block_keys(int r0, int r1, int Lq, int Lk, int wl, int wr) {
  KeyRange k;
  k.lo = band_lo(r0, Lq, Lk, wl);
  k.hi = band_hi(r1, Lq, Lk, wr);
  k.full_lo = band_lo(r1, Lq, Lk, wl);
  k.full_hi = band_hi(r0, Lq, Lk, wr);
  return k;
}

// Query rows that see some key of a key block [c0, c1] (inclusive, c1 < Lk),
// [lo, hi), and the rows that see every key of it, [full_lo, full_hi); rows
// clamped to [0, Lq]. Row i sees key j iff j - (Lk - Lq) - wr <= i <= j - (Lk - Lq) + wl.
struct RowRange {
  int lo, hi, full_lo, full_hi;
};
AV_HD inline int clamp_row(int64_t e, int Lq) { return e < 0 ? 0 : (e > Lq ? Lq : (int)e); }
AV_HD inline RowRange block_rows(int c0, int c1, int Lq, int Lk, int wl, int wr) {
  RowRange r;
  const int64_t off = (int64_t)Lk - Lq;
  r.lo = wr < 0 ? 0 : clamp_row(c0 - off - wr, Lq);
  r.hi = wl < 0 ? Lq : clamp_row(c1 - off + wl + 1, Lq);
  r.full_lo = wr < 0 ? 0 : clamp_row(c1 - off - wr, Lq);
  r.full_hi = wl < 0 ? Lq : clamp_row(c0 - off + wl + 1, Lq);
  return r;
}

// Tiles of a work item, in units of whole tiles: the tiles [lo, hi) that hold
// some visible (row, key) pair of the item, and among them [full_lo, full_hi)
// (empty when full_hi <= full_lo), the tiles whose every pair is visible, which
// the kernels run without a mask.
struct TileSpan {
  int lo, hi, full_lo, full_hi;
};

// Key tiles of bn keys met by the query rows [r0, r1] (inclusive, in range) of
// a query block. A partial last tile (keys past Lk) is never full.
AV_HD inline TileSpan key_tiles(int r0, int r1, int bn, int Lq, int Lk, int wl, int wr) {
  const KeyRange kr = block_keys(r0, r1, Lq, Lk, wl, wr);
  TileSpan t;
  t.lo = kr.lo / bn;
  t.hi = (kr.hi > kr.lo) ? ceil_div(kr.hi, bn) : t.lo;
  t.full_lo = t.lo > ceil_div(kr.full_lo, bn) ? t.lo : ceil_div(kr.full_lo, bn);
  t.full_hi = t.hi < kr.full_hi / bn ? t.hi : kr.full_hi / bn;
  return t;
}

// Query steps of bmq rows that meet the keys [c0, c1] (inclusive, in range) of
// a key block. Rows past Lq read as zero and add nothing to dK / dV, so a last
// partial step counts as full when every row of the sequence in it sees every
// key of the block.
AV_HD inline TileSpan query_steps(int c0, int c1, int bmq, int Lq, int Lk, int wl, int wr) {
  const RowRange rr = block_rows(c0, c1, Lq, Lk, wl, wr);
  TileSpan s;
  s.lo = rr.lo / bmq;
  s.hi = (rr.hi > rr.lo) ? ceil_div(rr.hi, bmq) : s.lo;
  s.full_lo = s.lo > ceil_div(rr.full_lo, bmq) ? s.lo : ceil_div(rr.full_lo, bmq);
  s.full_hi = (rr.full_hi >= Lq) ? s.hi : (s.hi < rr.full_hi / bmq ? s.hi : rr.full_hi / bmq);
  if (s.full_hi < s.full_lo) s.full_hi = s.full_lo;
  return s;
}

// With a left band edge, the forward splits an item's key tiles [t_lo, t_hi)
// (unmasked ones [f_lo, f_hi)) into: nh left-edge tiles that cross some row's
// left edge but lie left of every row's right edge, then unmasked tiles up to
// nm, then masked ones (local indices from t_lo). The left-edge tiles have
// their scores masked by the step before them and then take the unmasked
// probability path; that needs every row that reaches them to see at least a
// tile of keys, which a window of at least bn keys left of the diagonal gives.
// nh is even (the steady-state loop runs tiles in pairs); when the left-edge
// tiles do not end before the unmasked ones do, every tile runs masked
// (nh = nm = 0).
AV_HD inline void left_edge_tiles(int t_lo, int t_hi, int f_lo, int f_hi, int wl, int bn, int& nh, int& nm) {
  nh = 0;
  nm = 0;
  if (wl < bn) return;
  const int fe = f_hi < t_hi ? f_hi : t_hi;
  const int nme = fe - t_lo > 0 ? fe - t_lo : 0;
  int he = f_lo < f_hi ? f_lo : f_hi;
  he = he < t_hi ? he : t_hi;
  int hh = he - t_lo > 0 ? he - t_lo : 0;
  hh += hh & 1;
  if (hh < nme) {
    nh = hh;
    nm = nme;
  }
}

// Tile shapes of the kernels, shared with the host-side plan inspection: the
// forward and dQ kernels take query blocks of kQueryBlock rows against key
// tiles of key_tile(D) keys; the dK / dV kernels take key blocks of kKeyBlock
// keys against query steps of query_step(D) rows.
constexpr int kQueryBlock = 128;
constexpr int kKeyBlock = 128;
// Query heads per forward / dQ workgroup: the workgroup's four 32-row waves
// cover block_heads(r) heads of one KV group (r heads) and kQueryBlock /
// block_heads(r) rows of each. Grouping heads keeps the block's rows few, so a
// causal diagonal crosses fewer key tiles, while the waves still share every
// K / V tile.
AV_HD constexpr int block_heads(int r) { return r % 4 == 0 ? 4 : r % 2 == 0 ? 2 : 1; }
AV_HD constexpr int log2_small(int x) { return x >= 4 ? 2 : x >= 2 ? 1 : 0; }
AV_HD constexpr int key_tile(int D) { return D <= 128 ? 64 : 32; }
AV_HD constexpr int query_step(int D) { return D <= 128 ? 128 : 32; }

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
