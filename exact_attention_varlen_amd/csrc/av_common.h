// av_common.h — gfx950 device building blocks shared by the attention kernels:
// bf16 MFMA tile operations, bf16 conversion, wave-level exchanges, the
// work-item decode and the operand lane maps.
//
// MFMA used: v_mfma_f32_32x32x16_bf16 (D = A*B + C, A 32x16, B 16x32, fp32 C/D).
// Operand lanes: lane l supplies A row (l % 32) and B column (l % 32), each with
// 8 consecutive k values of k-group (l / 32). Result lanes: lane l, register v
// holds D[8*(v/4) + 4*(l/32) + (v%4)][l % 32].
//
// Row permutations used so that no operand needs an in-register shuffle:
//  * kperm(r): A-operand row r of the score product S^T = K * Q^T reads key
//    kperm(r) of the 32-key block. Then result register v of lane half h holds
//    key 16*(v/8) + 8*h + (v%8): registers 8s..8s+7 are 8 consecutive keys, which
//    is exactly the B-operand k-group of the next product (P^T as B operand)
//    for k-step s. Any consistent key order is exact, because the next product
//    sums over keys.
//  * dperm(r): A-operand row r of O^T = V^T * P^T reads head-dim row dperm(r).
//    Then result register v of lane half h holds head-dim 16*h + v, so each lane
//    stores 16 consecutive output values.
#ifndef AV_COMMON_H
#define AV_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_sched.h"

namespace av {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Round-to-nearest-even float -> bf16 of two values, packed (lo in bits 0..15):
// one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Eight fp32 values -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 to_bf16x8(float x0, float x1, float x2, float x3, float x4, float x5, float x6,
                                            float x7) {
  uint4 u;
  u.x = pack_bf16x2(x0, x1);
  u.y = pack_bf16x2(x2, x3);
  u.z = pack_bf16x2(x4, x5);
  u.w = pack_bf16x2(x6, x7);
  return as_bf16x8(u);
}

// Eight fp32 values -> bf16 parts hi + lo with x ~= hi + lo to about 16 bits of
// mantissa (lo is the bf16 rounding of the residual x - hi).
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint4 h, l;
  uint32_t* hw = reinterpret_cast<uint32_t*>(&h);
  uint32_t* lw = reinterpret_cast<uint32_t*>(&l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    hw[i] = w;
    const float r0 = x[2 * i] - __uint_as_float(w << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(w & 0xffff0000u);
    lw[i] = pack_bf16x2(r0, r1);
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// c + (sum of the two bf16 halves of w), one v_dot2 against (1, 1).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_bf16x2(uint32_t w, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), c,
                                         false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value of lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max(x, value of lane l ^ 32) without LDS traffic: v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second, so with
// both operands x every lane ends up holding its own value and its partner's.
__device__ __forceinline__ float max_xor32(float x) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// HBM -> LDS staging without VGPRs (buffer_load_dwordx4 ... lds): each lane of a
// wave moves 16 bytes to LDS address (m0 base + 16 * lane). Loads past the
// buffer's num_records return zeros, which bounds-checks the sequence tail.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, range-checked against num_bytes).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
  r[2] = (int)num_bytes;
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// One wave-wide 16-byte-per-lane copy HBM -> LDS at (lds_wave_base + 16 * lane).
// Written as inline assembly so that the compiler does not treat every later
// LDS read as aliasing the copy and wait for all copies in flight; the callers
// order the copies explicitly with wait_vmcnt() and lds_barrier(). The copy
// writes no VGPR. lds_wave_base must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const i32x4& rsrc, uint32_t lds_wave_base, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_wave_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  }
}

// Workgroup barrier that orders LDS accesses without the full memory fence of
// __syncthreads (which would also wait for every copy in flight). Outstanding
// LDS reads of this wave complete first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(const lds_char* p) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Transposing LDS read of 4 bf16 (ds_read_b64_tr_b16). Within each group of 16
// lanes, result element j of lane i is element (i % 4) of the 8 bytes addressed
// by lane 4 * j + i / 4: if lane 4j + c of the group addresses row (k0 + j),
// columns [4c, 4c + 4) of a row-major tile, lane i receives column i of rows
// k0 .. k0 + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr4(const lds_char* p) {
  const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<lds_char*>(p)));
  return __builtin_bit_cast(uint2, t);
}

// XOR swizzle of 16-byte chunks inside an LDS tile row (row r of a key tile):
// chunk c of row r is stored at chunk position c ^ swz(r). It makes the MFMA
// operand reads conflict-free: 16 consecutive rows read at one chunk hit 16
// distinct positions, and 4 consecutive rows read at 4 consecutive chunks (the
// transposed V reads) also hit 16 distinct positions. For head_dim 64 (two rows
// per 256-byte bank row) the map is chosen per row pair instead.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) {
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  } else {
    return 4 * (r & 3) + ((r >> 2) & 3);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int kperm(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
__device__ __forceinline__ int dperm(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// 16-byte loads/stores.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// ---------------------------------------------------------------------------
// Work-item decode: rank -> (sequence, query block), computed by one wave with
// all lanes agreeing on the result. See av_sched.h for the ranking.
// ---------------------------------------------------------------------------

// Number of blocks of sequence b (0 beyond num_seqs).
__device__ __forceinline__ int seq_blocks(const int32_t* cu, int b, int num_seqs, int bm) {
  if (b >= num_seqs) return 0;
  return ceil_div(cu[b + 1] - cu[b], bm);
}

// C(k) = sum_b max(0, nb_b - k), per lane for the lane's own k; up to 64
// sequences, nb_lane the block count of sequence `lane`.
__device__ __forceinline__ int count_at_least(int num_seqs, int nb_lane, int k) {
  int acc = 0;
  for (int bb = 0; bb < num_seqs; ++bb) {
    const int nb = __builtin_amdgcn_readlane(nb_lane, bb);
    acc += max(0, nb - k);
  }
  return acc;
}

__device__ __forceinline__ int highest_bit(uint64_t m) { return 63 - __builtin_clzll(m); }

// Up to 64 sequences. Returns false when `rank` is past the last block. Must be
// called by all 64 lanes of a wave (the counts are evaluated with every lane
// active so that the cross-lane reads see defined values). nb_lane is the block
// count of sequence `lane` (0 past the last sequence).
__device__ inline bool decode_rank_nb(int num_seqs, int levels, int rank, int nb_lane, int& b_out, int& m_out) {
  const int lane = threadIdx.x & (kWave - 1);
  if (levels <= 0) return false;
  // C(k) falls as k grows; the level of `rank` is the largest k < levels with
  // C(k) > rank. Pass 1: lane t probes k = t * stride.
  int stride = ceil_div(levels, kWave);
  const int k1 = lane * stride;
  const int c1 = count_at_least(num_seqs, nb_lane, k1);
  const uint64_t mask = __ballot((k1 < levels) && (c1 > rank));
  if (mask == 0) return false;
  int kstar = highest_bit(mask) * stride;
  // Then narrow the segment [kstar, kstar + stride), where C(kstar) > rank, by a
  // factor of 64 per pass until it is one level wide: lane t probes
  // kstar + t * sub. One pass when levels <= 4096 (block counts up to 2^12),
  // at most three more up to 2^24 levels.
  while (stride > 1) {
    const int sub = ceil_div(stride, kWave);
    const int k2 = kstar + lane * sub;
    const int c2 = count_at_least(num_seqs, nb_lane, k2);
    const uint64_t mask2 = __ballot((lane * sub < stride) && (k2 < levels) && (c2 > rank));
    kstar += highest_bit(mask2) * sub;  // lane 0 probes kstar itself, so mask2 != 0
    stride = sub;
  }
  // rank within level kstar: subtract the number of blocks of higher index
  const int above = count_at_least(num_seqs, nb_lane, kstar + 1);
  int j = rank - __builtin_amdgcn_readfirstlane(above);
  const uint64_t sel = __ballot(nb_lane > kstar);
  if (j >= __popcll(sel)) return false;
  // position of the (j+1)-th set bit
  uint64_t bits = sel;
  for (int i = 0; i < j; ++i) bits &= bits - 1;
  b_out = __builtin_ctzll(bits);
  m_out = kstar;
  return true;
}

// Sum over the wave's lanes, as a wave-uniform value (all 64 lanes active).
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return __builtin_amdgcn_readfirstlane(x);
}

// Exclusive prefix sum over the wave's lanes in lane order (all lanes active).
__device__ __forceinline__ int wave_excl_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
  int inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  return inc - x;
}

// Block counts of sequences first .. first + N - 1, 0 for those at or past
// `last` (last <= num_seqs). The loads are unconditional, their indices clamped
// to the array, so no lane-dependent branch is needed.
template <int N>
__device__ __forceinline__ void chunk_blocks(const int32_t* cu, int num_seqs, int bm, int first, int last,
                                             int (&nb)[N]) {
  int c[N + 1];
#pragma unroll
  for (int i = 0; i <= N; ++i) c[i] = cu[min(first + i, num_seqs)];
#pragma unroll
  for (int i = 0; i < N; ++i) nb[i] = (first + i < last) ? ceil_div(c[i + 1] - c[i], bm) : 0;
}

// More than 64 sequences. Lane t owns the consecutive sequences
// [t S, (t + 1) S), S = ceil(num_seqs / 64), and holds the block counts of the
// first kDecodeChunk of them in registers (the rest are reloaded in rounds of
// that size for each pass over them). C(k) is a wave sum of the lanes' partial
// counts, the level of `rank` is found by bisection over k (one pass per step),
// and the sequence by a prefix count of each lane's sequences at that level (one
// pass that also forms C(level + 1), one that picks): O(S log(levels)) per wave,
// instead of O(num_seqs) per probe. Same ranking and contract as decode_rank_nb.
constexpr int kDecodeChunk = 16;
__device__ inline bool decode_rank_many(const int32_t* cu, int num_seqs, int bm, int levels, int rank, int& b_out,
                                        int& m_out) {
  const int lane = threadIdx.x & (kWave - 1);
  if (levels <= 0) return false;
  const int S = ceil_div(num_seqs, kWave);
  const int rounds = ceil_div(S, kDecodeChunk);
  const int first = lane * S, last = min(first + S, num_seqs);
  int held[kDecodeChunk];
  chunk_blocks(cu, num_seqs, bm, first, last, held);
  // f(nb) for each of this lane's sequences (nb = 0 past the end of its chunk)
  auto lane_pass = [&](auto f) {
#pragma unroll
    for (int i = 0; i < kDecodeChunk; ++i) f(held[i]);
    for (int r = 1; r < rounds; ++r) {
      int nb[kDecodeChunk];
      chunk_blocks(cu, num_seqs, bm, first + r * kDecodeChunk, last, nb);
#pragma unroll
      for (int i = 0; i < kDecodeChunk; ++i) f(nb[i]);
    }
  };
  // The level: the largest k < levels with C(k) > rank (C falls as k grows),
  // by bisection that keeps C(hi) <= rank or hi == levels. When rank is past the
  // last block (C(0) <= rank) it ends at k = 0 with no sequence left to pick.
  int lo = 0, hi = levels;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    int acc = 0;
    lane_pass([&](int nb) { acc += max(0, nb - mid); });
    if (wave_sum(acc) > rank) lo = mid;
    else hi = mid;
  }
  const int kstar = lo;
  // one pass: C(kstar + 1), and this lane's sequences with more than kstar blocks
  int above = 0, own = 0;
  lane_pass([&](int nb) {
    above += max(0, nb - kstar - 1);
    own += nb > kstar ? 1 : 0;
  });
  // rank within level kstar, then the (j+1)-th sequence with more than kstar blocks
  const int j = rank - wave_sum(above);
  const int before = wave_excl_scan(own);
  const uint64_t owner_mask = __ballot(j >= before && j < before + own);
  if (owner_mask == 0) return false;
  const int owner = __builtin_ctzll(owner_mask);
  // each lane picks the (j - before + 1)-th of its sequences at this level; only
  // the owner's pick is taken
  int want = j - before, b = -1;
  auto pick = [&](const int (&nb)[kDecodeChunk], int base) {
#pragma unroll
    for (int i = 0; i < kDecodeChunk; ++i) {
      const int hit = nb[i] > kstar ? 1 : 0;
      b = (hit && want == 0) ? base + i : b;
      want -= hit;
    }
  };
  pick(held, first);
  for (int r = 1; r < rounds; ++r) {
    int nb[kDecodeChunk];
    chunk_blocks(cu, num_seqs, bm, first + r * kDecodeChunk, last, nb);
    pick(nb, first + r * kDecodeChunk);
  }
  b_out = __builtin_amdgcn_readlane(b, owner);
  m_out = kstar;
  return b_out >= 0;
}

// rank -> (sequence, block) for any number of sequences.
__device__ inline bool decode_rank(const int32_t* cu, int num_seqs, int bm, int levels, int rank, int& b_out,
                                   int& m_out) {
  const int lane = threadIdx.x & (kWave - 1);
  if (num_seqs > kWave) return decode_rank_many(cu, num_seqs, bm, levels, rank, b_out, m_out);
  return decode_rank_nb(num_seqs, levels, rank, seq_blocks(cu, lane, num_seqs, bm), b_out, m_out);
}

// A decoded work item: sequence b, block m of its ranked rows, and the
// sequence's query rows [cq, cq + Lq) and key rows [ck, ck + Lk).
struct Item {
  int b, m, cq, Lq, ck, Lk;
};

// decode_rank plus the chosen sequence's bounds, ranking blocks of bm query
// rows, or of key rows with BY_KEYS. With up to 64 sequences every lane loads
// its own sequence's four bounds at once, the decode works from them, and the
// item's bounds are read from lane b: no memory round trip follows the decode.
template <bool BY_KEYS>
__device__ inline bool decode_item(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int bm, int levels,
                                   int rank, Item& it) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t* cu = BY_KEYS ? cu_k : cu_q;
  if (num_seqs <= kWave) {
    int q0 = 0, q1 = 0, k0 = 0, k1 = 0;
    if (lane < num_seqs) {
      q0 = cu_q[lane];
      q1 = cu_q[lane + 1];
      k0 = cu_k[lane];
      k1 = cu_k[lane + 1];
    }
    const int nb = ceil_div(BY_KEYS ? k1 - k0 : q1 - q0, bm);
    if (!decode_rank_nb(num_seqs, levels, rank, nb, it.b, it.m)) return false;
    const int b = __builtin_amdgcn_readfirstlane(it.b);
    it.cq = __builtin_amdgcn_readlane(q0, b);
    it.Lq = __builtin_amdgcn_readlane(q1, b) - it.cq;
    it.ck = __builtin_amdgcn_readlane(k0, b);
    it.Lk = __builtin_amdgcn_readlane(k1, b) - it.ck;
    return true;
  }
  if (!decode_rank(cu, num_seqs, bm, levels, rank, it.b, it.m)) return false;
  it.cq = cu_q[it.b];
  it.Lq = cu_q[it.b + 1] - it.cq;
  it.ck = cu_k[it.b];
  it.Lk = cu_k[it.b + 1] - it.ck;
  return true;
}

}  // namespace av

#endif  // AV_COMMON_H
