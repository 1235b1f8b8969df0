// tile_io.h -- bf16 tiles of [rows][D] (D contiguous in HBM) in LDS.
//
// Tiles are copied from HBM straight into LDS with buffer loads that write
// LDS directly (no staging registers).  The buffer resource of a tile
// covers exactly the rows of its half, so rows past the end of the half
// read as zero.  In LDS a tile is row-major with no padding; the 16-byte
// chunk c of row r sits at chunk c ^ swz(r).  swz permutes the chunks of
// every group of consecutive rows so that two read patterns are free of
// bank conflicts (64 banks of 4 bytes):
//  * natural operand reads: 8 consecutive rows, one 16-byte chunk each
//    (ds_read_b128), e.g. K as the A operand of S^T = K Q^T;
//  * transposing reads (ds_read_b64_tr_b16): a 16-lane group reads 4
//    consecutive rows x 16 columns (two chunks per row) and every lane
//    receives the 4 rows of one column.  swz maps the 4 rows to 4 disjoint
//    chunk pairs.  This yields operands contracted over the tile's rows
//    (V^T for O^T = V^T P^T, dO^T and Q^T for dV^T, dK^T, K^T for dQ^T)
//    from the same natural tile.
#pragma once

#include "common.h"

namespace bd {

//
// The right permutation depends on where a row starts among the banks.  A
// row of D bf16 is D / 2 dwords:
//  * D = 128, 256 (a multiple of 64 dwords): every row starts on bank 0, so
//    16 consecutive rows need 16 distinct chunk positions: a permutation of
//    0..15 (the 4-row groups of a transposing read land on distinct
//    quarters of the banks through the high two bits);
//  * D = 64, 192 (32 mod 64 dwords): odd rows start half-way along the
//    banks, so 3 bits suffice, and they keep every chunk inside its
//    aligned group of 8 (D = 192 rows hold 24 chunks);
//  * D = 96 (48 mod 64 dwords): the 4 rows of a transposing read already
//    start on 4 distinct quarters of the banks; rows 4 apart share a
//    quarter and are separated by a 2-bit permutation, which keeps every
//    chunk inside its aligned group of 4 (rows of 12 chunks).
template <int D>
__device__ __forceinline__ int swz(int row) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dimension");
  if constexpr (D == 128 || D == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  if constexpr (D == 96) return (row >> 2) & 3;
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// The chunks swz permutes: chunk c ^ swz(r) stays in c's aligned group of
// this many chunks, so chunks SPAN apart sit SPAN * 8 elements apart in
// every row.  Per-lane offset tables therefore need one entry per position
// in the group; the rest is a compile-time offset (an immediate of the LDS
// instruction).
template <int D>
constexpr int swz_span() {
  return D == 96 ? 4 : (D == 128 || D == 256) ? 16 : 8;
}

template <int D>
__device__ __forceinline__ int nat_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}

// 8 elements (16 bytes) of row `row`, chunk `chunk`.
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* t, int row, int chunk) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(t + nat_off<D>(row, chunk)));
}

// Transposing read of rows [row0, row0 + 4) (row0 % 4 == 0) and columns
// [col0, col0 + 16) (col0 % 16 == 0) by the 16-lane group of this lane:
// lane i of the group receives column col0 + i of the 4 rows.
template <int D>
__device__ __forceinline__ bf16x4 lds_tr4(const uint16_t* t, int row0, int col0, int lane) {
  const int s = lane & 15;
  const int row = row0 + (s >> 2);
  const int col = col0 + 4 * (s & 3);
  const uint16_t* p = t + nat_off<D>(row, col >> 3) + (col & 7);
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// A operand of a 32x32x16 product contracted over tile rows: lane (l32, h2)
// gets column col_base + l32 at rows rbase + 4h2 + {0..3} and
// rbase + 8 + 4h2 + {0..3} -- the row order of the D-layout registers that
// form the matching B operand (common.h).
template <int D>
__device__ __forceinline__ bf16x8 lds_trA(const uint16_t* t, int rbase, int col_base, int lane) {
  const int l32 = lane & 31, h2 = lane >> 5;
  const int col0 = col_base + (l32 & 16);
  bf16x4 lo = lds_tr4<D>(t, rbase + 4 * h2, col0, lane);
  bf16x4 hi = lds_tr4<D>(t, rbase + 8 + 4 * h2, col0, lane);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same two reads with the lane's part of the address precomputed: the
// kernels keep these per-lane offsets (elements) in registers for the whole
// walk, so that inside the loops every read is a register plus a
// compile-time offset (whole 16-row steps leave swz unchanged).
template <int D>
__device__ __forceinline__ int row8_lane_off(int lane, int chunk_base) {
  return nat_off<D>(lane & 31, chunk_base + (lane >> 5));
}

template <int D>
__device__ __forceinline__ int trA_lane_off(int lane, int col_base, int upper) {
  const int l32 = lane & 31, h2 = lane >> 5, s = lane & 15;
  const int row = 8 * upper + 4 * h2 + (s >> 2);
  const int col = col_base + (l32 & 16) + 4 * (s & 3);
  return nat_off<D>(row, col >> 3) + (col & 7);
}

__device__ __forceinline__ bf16x8 lds_vec_at(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 lds_trA_at(const uint16_t* lo, const uint16_t* hi) {
  bf16x4 a = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (__attribute__((address_space(3))) shortx4*)(lo)));
  bf16x4 b = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (__attribute__((address_space(3))) shortx4*)(hi)));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Copy rows [row0, row0 + ROWS) of a [n][D] view (row stride row_bytes) into
// an LDS tile, NT threads cooperating; each lane writes 16 bytes and every
// wave-wide instruction fills 1 KiB of consecutive LDS.
template <int ROWS, int D, int NT>
struct DirectTile {
  static constexpr int CH = D / 8;
  static constexpr int SLOTS = ROWS * CH;
  static constexpr int PER = (SLOTS + NT - 1) / NT;
  static constexpr int ELEMS = ROWS * D;
  // whole waves: the last pass, when partial, is skipped by entire waves
  static_assert(SLOTS % 64 == 0 && NT % 64 == 0, "tile must split into whole waves");

  // lds: LDS byte address of the tile (lds_byte_addr)
  __device__ __forceinline__ static void load(rsrc_t src, uint32_t row_bytes, int row0, uint32_t lds,
                                              int tid) {
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (SLOTS % NT != 0 && i == PER - 1 && i * NT + wbase >= SLOTS) break;
      const int slot = i * NT + tid;
      const int r = slot / CH;
      const int c = (slot % CH) ^ swz<D>(r);
      const uint32_t voff = (uint32_t)r * row_bytes + (uint32_t)c * 16u;
      lds_direct16(src, lds + (uint32_t)(i * NT + wbase) * 16u, voff, (uint32_t)row0 * row_bytes);
    }
  }
};

}  // namespace bd
