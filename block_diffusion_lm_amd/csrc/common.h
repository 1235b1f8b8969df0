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

#include <type_traits>

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

// acc + the sum of eight bf16 values (exact products with 1.0, float32
// accumulation): four v_dot2c_f32_bf16 against the pair (1, 1).
__device__ __forceinline__ float sum_bf16x8(const bf16x8& x, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
  return acc;
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

// Issue priority of the wave around a burst of MFMAs (compiled in with
// BDATTN_SETPRIO).  A wave's own vector ALU work does not overlap its MFMAs
// (measured on MI355X), so throughput comes from the other wave on the SIMD
// running its softmax arithmetic meanwhile; raising the priority of the wave
// in an MFMA burst was meant to keep the matrix core fed, but measured 3-5%
// slower in every kernel, so it is off by default.
#ifdef BDATTN_SETPRIO
__device__ __forceinline__ void mfma_burst_begin() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_burst_end() { __builtin_amdgcn_s_setprio(0); }
#else
__device__ __forceinline__ void mfma_burst_begin() {}
__device__ __forceinline__ void mfma_burst_end() {}
#endif

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

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Buffer loads that write LDS directly.  The wave's 64 lanes fill
// consecutive LDS from lds_wave, the wave's LDS byte address (uniform), 16
// or 4 bytes per lane.
//
// They are issued from inline assembly that sets M0 (the LDS base) itself.
// The compiler's own form of this load makes every later transposing LDS
// read (ds_read_b64_tr_b16) wait until all such loads in flight have landed,
// wherever they write, which would stall each tile's products on the load
// of the next tile.  The kernels order these loads explicitly instead: an
// LDS buffer is read only after wait_vmem() and a workgroup barrier, and
// refilled only after the barrier that follows its last reads.  No other
// code in these kernels keeps a value in M0.
//
// Debug build (BDATTN_LDS_POISON): before each such load, every lane first
// writes NaN over exactly the LDS bytes its load will fill and waits for
// that write.  A load is only issued once every read of the buffer's old
// contents is over, so a read that comes too late (after the refill was
// issued) or too early (before the new tile landed) sees NaN instead of
// plausible stale data, and the results turn to NaN.
#ifdef BDATTN_LDS_POISON
__device__ __forceinline__ void lds_poison(uint32_t lds_wave, uint32_t bytes_per_lane) {
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const uint32_t addr = lds_wave + lane * bytes_per_lane;
  if (bytes_per_lane == 16) {
    const u32x4 nan4 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)addr = nan4;
  } else {
    *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)addr = 0x7fc00000u;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
#endif

__device__ __forceinline__ void lds_direct16(rsrc_t r, uint32_t lds_wave, uint32_t voff, uint32_t soff) {
#ifdef BDATTN_LDS_POISON
  lds_poison(lds_wave, 16);
#endif
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(soff), "s"(lds_wave)
      : "memory");
}

__device__ __forceinline__ void lds_direct4(rsrc_t r, uint32_t lds_wave, uint32_t voff, uint32_t soff) {
#ifdef BDATTN_LDS_POISON
  lds_poison(lds_wave, 4);
#endif
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(soff), "s"(lds_wave)
      : "memory");
}

// Makes the compiler complete a register load here rather than at the
// register's first use.  When that use sits inside a tile loop the wait it
// places there also covers the loads into LDS issued in the loop (the
// counter is shared), which would stall every iteration on the next tile.
template <typename T>
__device__ __forceinline__ void settle(T& v) {
  asm volatile("" : "+v"(v));
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled at compile
// time (for code whose indices must be constants, such as LDS buffer
// numbers that become immediate address offsets).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Wait until this wave's loads into LDS (and all its other vector memory
// loads) have landed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most `keep` tiles of this wave's tile loads (PER load
// instructions each, issued in tile order) are still in flight: the oldest
// tiles have landed.  keep is uniform, 0 <= keep <= MAXKEEP.
template <int MAXKEEP, int PER>
__device__ __forceinline__ void wait_tiles(int keep) {
  if constexpr (MAXKEEP >= 2) {
    if (keep >= 2) { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER) : "memory"); return; }
  }
  if constexpr (MAXKEEP >= 1) {
    if (keep >= 1) { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); return; }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

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
