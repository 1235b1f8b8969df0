// common.h -- types and wave-level helpers for the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (CDNA4, wave64,
// v_mfma_f32_32x32x16_bf16, D = A * B + C with A 32x16, B 16x32):
//   A operand : lane l holds A[row = l % 32][k = 8 * (l / 32) + j], j = 0..7
//   B operand : lane l holds B[k = 8 * (l / 32) + j][col = l % 32]
//   D result  : lane l, register r (0..15) holds
//               D[row = 8 * (r / 4) + 4 * (l / 32) + r % 4][col = l % 32]
// Only the pairing of A's and B's k index matters for a contraction, so the
// kernels are free to permute which k each (lane half, j) slot stands for,
// as long as both operands agree.  The kernels exploit this: the result of
// one product, read with k = its row index, is directly a valid B operand
// (or, transposed, a valid A operand) of the next product, with the row
// permutation of the D layout, so scores never leave registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Eight consecutive float32 values rounded (to nearest even) to bf16.
__device__ __forceinline__ bf16x8 pack_bf16x8(const floatx16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[base + j];
  return r;
}

// Reductions between lane l and lane l ^ 32.  v_permlane32_swap with the
// same register as both operands leaves, in every lane, its own value in one
// result and the other half's value in the other; combining both results
// is therefore independent of which result holds which.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros (the hardware range check), which is how ragged tiles are padded.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ float buf_ldf(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: the wave's 64 lanes
// fill 1 KiB starting at lds_wave (which must be the same for the wave).
__device__ __forceinline__ void lds_direct16(rsrc_t r, uint16_t* lds_wave, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave, 16, voff, soff, 0, 0);
}

// 4 bytes per lane straight into LDS (256 bytes per wave).
__device__ __forceinline__ void lds_direct4(rsrc_t r, void* lds_wave, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave, 4, voff, soff, 0, 0);
}

// Wait until this wave's loads into LDS (and all its other vector memory
// loads) have landed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte global load / store helpers (bf16 stored as raw 16-bit words).
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Position of tile-local key kappa in a key-contiguous ("transposed") LDS
// row.  Within every group of 16 keys the 4-key groups are stored in the
// order 0, 2, 1, 3, so that the 8 keys a lane half needs for one MFMA
// k-step (keys 4h..4h+3 and 8+4h..8+4h+3, the D-layout row permutation)
// are 8 consecutive elements: one 16-byte LDS read.
__device__ __forceinline__ int tpos(int kappa) {
  int g4 = (kappa >> 2) & 3;
  int slot = ((g4 & 1) << 1) | (g4 >> 1);  // 0->0, 1->2, 2->1, 3->3
  return (kappa & ~15) | (slot << 2) | (kappa & 3);
}

}  // namespace bd
