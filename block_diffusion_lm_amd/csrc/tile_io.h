// tile_io.h -- moving bf16 tiles of [rows][D] (D contiguous in HBM) into LDS.
//
// Two LDS layouts are produced from one global read:
//  * natural:    [rows][D], no padding; the 16-byte chunk c of a row r is
//                stored at chunk c ^ swz(r).  Both the MFMA operand reads
//                (8 consecutive rows, same chunk) and the stores of this
//                loader (rows 4g + j for 8 consecutive g) then hit 8
//                different 16-byte bank groups.
//  * transposed: [D][rows + 8], rows contiguous, in the order tpos()
//                (common.h), so that an MFMA operand whose contraction runs
//                over the rows is one 16-byte read per lane.
//
// Thread unit u covers 4 consecutive rows (4g .. 4g + 3) of one 8-element
// chunk c, with g varying fastest across lanes: a transposed store of a
// wave then fills one contiguous run of an LDS row.
#pragma once

#include "common.h"

namespace bd {

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }

template <int D>
__device__ __forceinline__ const uint16_t* nat_ptr(const uint16_t* lds, int row, int chunk) {
  return lds + row * D + ((chunk ^ swz(row)) << 3);
}

template <int D>
__device__ __forceinline__ bf16x8 lds_nat(const uint16_t* lds, int row, int chunk) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(nat_ptr<D>(lds, row, chunk)));
}

__device__ __forceinline__ bf16x8 lds_vec(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

template <int ROWS, int D, int NTHREADS>
struct TileLoader {
  static constexpr int G = ROWS / 4;
  static constexpr int C = D / 8;
  static constexpr int UNITS = G * C;
  static constexpr int PER = (UNITS + NTHREADS - 1) / NTHREADS;
  static constexpr int T_STRIDE = ROWS + 8;
  static constexpr int NAT_ELEMS = ROWS * D;
  static constexpr int T_ELEMS = D * T_STRIDE;

  u32x4 v[PER][4];

  __device__ __forceinline__ static bool active(int u) { return (UNITS % NTHREADS == 0) || u < UNITS; }

  // base: element (row 0, dim 0) of the tile's half for this head; rs: the
  // token stride in elements; rows >= nvalid (past the end of the half) are
  // read as zeros.
  __device__ __forceinline__ void load(const uint16_t* base, size_t rs, int row0, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + NTHREADS * i;
      if (!active(u)) continue;
      int g = u % G, c = u / G;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int row = row0 + 4 * g + j;
        v[i][j] = (row < nvalid) ? ld16(base + (size_t)row * rs + c * 8) : zero_u32x4();
      }
    }
  }

  __device__ __forceinline__ void store_nat(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + NTHREADS * i;
      if (!active(u)) continue;
      int g = u % G, c = u / G;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int row = 4 * g + j;
        *reinterpret_cast<u32x4*>(lds + row * D + ((c ^ swz(row)) << 3)) = v[i][j];
      }
    }
  }

  __device__ __forceinline__ void store_t(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + NTHREADS * i;
      if (!active(u)) continue;
      int g = u % G, c = u / G;
      int pos = tpos(4 * g);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t a0 = v[i][0][w], a1 = v[i][1][w], a2 = v[i][2][w], a3 = v[i][3][w];
        // dimension 8c + 2w: low 16 bits of each row's word
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        // dimension 8c + 2w + 1: high 16 bits
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *reinterpret_cast<u32x2*>(lds + (8 * c + 2 * w) * T_STRIDE + pos) = lo;
        *reinterpret_cast<u32x2*>(lds + (8 * c + 2 * w + 1) * T_STRIDE + pos) = hi;
      }
    }
  }
};

}  // namespace bd
