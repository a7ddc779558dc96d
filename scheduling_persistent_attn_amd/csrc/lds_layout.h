// Swizzled LDS layout for bf16 tiles whose rows are 128 or 256 bytes long.
//
// A tile is stored row-major in 256-byte "super-rows": a row of 256 bytes is
// one super-row; rows of 128 bytes are paired (row r is the half r & 1 of
// super-row r >> 1).  Each super-row holds 16 slots of 16 bytes and logical
// slot U of super-row R sits at slot U ^ sw(R).  The LDS of gfx950 serves
// 256 bytes per cycle from 64 four-byte banks; with
//   sw(R) = ((a << 1) ^ (a << 2)) ^ b,  a = R & 3,
//   b = (R >> 2) & 3 for 256-byte rows, 3 * ((R >> 2) & 1) for 128-byte rows,
// three access shapes are free of bank conflicts: 16-byte reads of one
// column in 16 consecutive rows, the transposing 8-byte reads
// (ds_read_b64_tr_b16) of 4 consecutive rows x 64 bytes, and those of two
// 4-row groups 8 rows apart x 32 bytes (each 32 lanes of such a read cover
// all 64 banks once).  For 128-byte rows the last shape is why b moves slot
// bits 0 and 1: with bit 0 alone, super-rows R and R ^ 4 fall on the same
// banks there.  sw depends only on the low bits of the row, so moving by 16
// rows is a constant offset, and moving a slot index by a multiple of 2 (a
// 32-byte step) is an XOR.
#pragma once

namespace dash {

__device__ __forceinline__ int lds_sw16(int R, int row_bytes) {
  const int a = R & 3;
  const int b = row_bytes == 256 ? ((R >> 2) & 3) : 3 * ((R >> 2) & 1);
  return ((a << 1) ^ (a << 2)) ^ b;
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a tile with RB-byte rows.
template <int RB>
__device__ __forceinline__ int lds_phys(int row, int chunk) {
  static_assert(RB == 128 || RB == 256, "row length");
  if constexpr (RB == 256) {
    return row * 256 + ((chunk ^ lds_sw16(row, 256)) << 4);
  } else {
    const int R = row >> 1;
    const int U = ((row & 1) << 3) | chunk;
    return R * 256 + ((U ^ lds_sw16(R, 128)) << 4);
  }
}

// Inverse, for the loaders: physical slot `slot` of super-row R holds 16-byte
// chunk *chunk of row *row.
template <int RB>
__device__ __forceinline__ void lds_slot_source(int R, int slot, int* row, int* chunk) {
  static_assert(RB == 128 || RB == 256, "row length");
  if constexpr (RB == 256) {
    *row = R;
    *chunk = slot ^ lds_sw16(R, 256);
  } else {
    const int U = slot ^ lds_sw16(R, 128);
    *row = 2 * R + (U >> 3);
    *chunk = U & 7;
  }
}

}  // namespace dash
