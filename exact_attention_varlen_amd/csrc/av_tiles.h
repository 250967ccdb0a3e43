// av_tiles.h — row tiles staged HBM -> LDS by buffer-load DMA, shared by the
// forward, dQ and dK/dV kernels.
//
// A tile is R rows of one head (head_dim D, bf16) of a (tokens, heads, D)
// tensor, stored row-major in LDS (D * 2 bytes per row) with the 16-byte chunk
// swizzle swz<D>. It is filled by R * D * 2 / 1024 wave-wide 1 KB copies; rows
// past the buffer's range read as zero. The same per-lane LDS offsets serve
// every tile of a given D:
//  * row_off[kk]   A operand of a product contracting over head_dim: lane l
//                  reads row kperm(l % 32) of a 32-row block, head-dims
//                  16 kk + 8 (l / 32) .. + 7 (16 bytes);
//  * tr_off0/1[db] A operand of a product contracting over rows: transposing
//                  reads of 4 rows x 4 head-dims; with tr_off0 for the first
//                  four k-slots and tr_off1 for the last four, lane l of the
//                  MFMA operand holds head-dim row (l % 32) of block db and the
//                  rows 16 s + 8 (l / 32) + 0..7 for k-step s (add 16 s rows).
#ifndef AV_TILES_H
#define AV_TILES_H

#include "av_common.h"

namespace av {

template <int D, int R>
struct RowTile {
  static constexpr int ROW = D * 2;                // bytes per row
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int BYTES = R * ROW;            // bytes of the tile
  static constexpr int DMAS = BYTES / 1024;        // wave-wide copies per tile
  static constexpr int ROWS_PER_DMA = 1024 / ROW;  // rows per copy
  static_assert(BYTES % 1024 == 0, "tile must be a whole number of 1 KB copies");
};

// Copy number `blk` (0 .. DMAS-1) of a tile whose first row is `row0` in the
// buffer, into the tile at LDS byte address `tile`.
template <int D, int R>
__device__ __forceinline__ void tile_dma(uint32_t tile, const i32x4& rsrc, uint32_t pitch, int row0, int blk,
                                         int lane) {
  using T = RowTile<D, R>;
  const int row = blk * T::ROWS_PER_DMA + lane / T::CPR;
  const int c = (lane % T::CPR) ^ swz<D>(row);
  const uint32_t voff = (uint32_t)(row0 + row) * pitch + (uint32_t)c * 16u;
  lds_dma16(rsrc, tile + blk * 1024, voff);
}

// Buffer descriptor of `rows` rows of one head: rows past the end read as 0.
template <int D>
__device__ __forceinline__ i32x4 head_rows_rsrc(const uint16_t* first_row_head, int rows, uint32_t pitch) {
  const uint32_t nbytes = (rows > 0) ? (uint32_t)(rows - 1) * pitch + D * 2 : 0u;
  return make_rsrc(first_row_head, nbytes);
}

// Only the offsets of the first 16 chunks of a row are stored: the swizzle
// changes the low 4 bits of a chunk index only, so chunk c + 16 lies 256 bytes
// after chunk c (head_dim 256 has 32 chunks per row). row(kk) and tr(db) add
// that part as an immediate.
template <int D>
struct OperandOffsets {
  static constexpr int NR = (D / 16 < 8) ? D / 16 : 8;
  static constexpr int NT = (D / 32 < 4) ? D / 32 : 4;
  uint32_t row_off[NR];
  uint32_t tr_off0[NT];
  uint32_t tr_off1[NT];
  __device__ __forceinline__ uint32_t row(int kk) const { return row_off[kk % NR] + 256u * (kk / NR); }
  __device__ __forceinline__ uint32_t tr0(int db) const { return tr_off0[db % NT] + 256u * (db / NT); }
  __device__ __forceinline__ uint32_t tr1(int db) const { return tr_off1[db % NT] + 256u * (db / NT); }
};

template <int D>
__device__ __forceinline__ void operand_offsets(OperandOffsets<D>& o, int lane) {
  constexpr int ROW = D * 2;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int row = kperm(col);
#pragma unroll
  for (int kk = 0; kk < OperandOffsets<D>::NR; ++kk) o.row_off[kk] = row * ROW + (((2 * kk + half) ^ swz<D>(row)) << 4);
  const int grp = lane >> 4;  // 16-lane group: head-dim half (grp & 1) and k-group (grp >> 1)
  const int i = lane & 15;
  const int j = i >> 2;  // row within the 4-row read
  const int cc = i & 3;  // 4-column piece
  const int r0 = 8 * half + j;
  const int r1 = r0 + 4;
#pragma unroll
  for (int db = 0; db < OperandOffsets<D>::NT; ++db) {
    const int chunk = db * 4 + 2 * (grp & 1) + (cc >> 1);
    o.tr_off0[db] = r0 * ROW + ((chunk ^ swz<D>(r0)) << 4) + (cc & 1) * 8;
    o.tr_off1[db] = r1 * ROW + ((chunk ^ swz<D>(r1)) << 4) + (cc & 1) * 8;
  }
}

// Transposed operand (head-dim block db, rows rows0 .. rows0 + 15 of the tile
// at `tile`, where rows0 = 16 s for k-step s of a 32-row block).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const lds_char* rows0, const OperandOffsets<D>& o, int db) {
  const uint2 lo = lds_read_tr4(rows0 + o.tr0(db));
  const uint2 hi = lds_read_tr4(rows0 + o.tr1(db));
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Store a 32 x 32 fp32 accumulator block (result of a transposed-operand
// product: register v of lane l is head-dim 8 (v / 4) + 4 (l / 32) + v % 4 of
// block db, for the row of column l % 32) as bf16, scaled.
__device__ __forceinline__ void store_acc_row(uint16_t* row_db, const f32x16& a, float scale) {
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    uint2 w;
    w.x = pack_bf16x2(a[4 * gq + 0] * scale, a[4 * gq + 1] * scale);
    w.y = pack_bf16x2(a[4 * gq + 2] * scale, a[4 * gq + 3] * scale);
    *reinterpret_cast<uint2*>(row_db + 8 * gq) = w;
  }
}

// The same block stored as fp32, unscaled / scaled (partial results).
__device__ __forceinline__ void store_acc_row_f32(float* row_db, const f32x16& a, float scale = 1.f) {
#pragma unroll
  for (int gq = 0; gq < 4; ++gq)
    *reinterpret_cast<float4*>(row_db + 8 * gq) =
        make_float4(a[4 * gq] * scale, a[4 * gq + 1] * scale, a[4 * gq + 2] * scale, a[4 * gq + 3] * scale);
}

}  // namespace av

#endif  // AV_TILES_H
