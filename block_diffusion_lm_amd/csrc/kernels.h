// kernels.h -- argument block and launchers of the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "geometry.h"

namespace bd {

struct AttnArgs {
  // inputs, bf16: q [B][T][H][D], k and v [B][T][Hkv][D] (packed samples:
  // [total][H][D] and [total][Hkv][D])
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;     // forward output, read by the backward
  const uint16_t* dout;  // gradient of the output
  // forward outputs
  uint16_t* out;
  float* lse;            // [B][H][T] (packed: [H][total]), natural log
  // backward
  const float* lse_in;   // [B][H][T]
  float* ndelta;         // workspace [B][H][T]: -(dout_i . out_i)
  float* lse2;           // workspace [B][H][T]: lse * log2(e)
  // FP8 forward: float32 descale factors of q [B][H], k and v [B][Hkv]
  const float* qd;
  const float* kd;
  const float* vd;
  uint16_t* dq;
  uint16_t* dk;   // [B][T][Hkv][D], like k
  uint16_t* dv;
  // packed samples: B + 1 token offsets in device memory (sample b holds
  // tokens [cu[b], cu[b+1])), or null for the batched layout
  const int* cu;
  long long tokens;   // tokens of all samples: B * T, or the packed total
  long long stat_hs;  // distance between heads in lse and the statistics: T, or the total
  // shape
  int B, H;
  int Hkv;      // key/value heads; query head h reads key/value head h / G
  int G;        // H / Hkv, query heads per key/value head
  int S;        // dK/dV workgroups per group of query heads (divides G)
  float* part;  // S > 1: float32 partial dK then dV, each [S][B][T][Hkv][D]
  int n;        // half length (diffusion) or sequence length (causal); packed: the longest
  int b;        // block size (1 for causal)
  int mode;     // MODE_DIFFUSION / MODE_CAUSAL
  int T;        // tokens per sample: 2n or n
  int nhalves;  // 2 or 1
  float scale;       // multiplies q.k (may be negative)
  float scale_log2;  // scale * log2(e)
  float softcap;     // > 0: scaled scores s become softcap * tanh(s / softcap); 0: off
};

// Query-stationary grids enumerate (sample, query head) pairs as
// x = gi * (B * Hkv) + bi * Hkv + hk with query head hh = hk * G + gi.  The G
// query heads that read one key/value head then sit B * Hkv blocks apart:
// the same residue modulo the XCD count when B * Hkv is a multiple of 8, so
// they share the L2 that holds that head's K and V.  With G = 1 this is
// x = bi * H + hh.
__device__ __forceinline__ void query_head(const AttnArgs& a, int x, int& bi, int& hh, int& hk) {
  const int BHkv = a.B * a.Hkv;
  const int gi = x / BHkv;
  const int r = x - gi * BHkv;
  bi = r / a.Hkv;
  hk = r - bi * a.Hkv;
  hh = hk * a.G + gi;
}

// How many workgroups the dK/dV kernel spreads each group of G query heads
// over: 1 (one workgroup walks the whole group) unless that leaves fewer
// than a few workgroups per CU; then the smallest divisor of G that does
// not.  Above 1 the workgroups write float32 partials that a reduction sums.
int dkdv_group_splits(int B, int n, int nhalves, int Hkv, int G, int D);

// Sample bi: the token index of its first token, its half length n
// (sequence length in causal mode) and the index of its statistics for
// head 0, row 0.  Batched: tok0 = bi * T, n = a.n, stat0 = bi * H * T.
// Packed: tok0 = stat0 = cu[bi] and n from cu[bi + 1] - cu[bi].  A packed
// sample whose offsets are inconsistent (negative, decreasing, past the
// packed total, an odd diffusion length, or a half longer than a.n) yields
// false, and its workgroups do nothing, so no access leaves the tensors.
__device__ __forceinline__ bool sample_of(const AttnArgs& a, int bi, size_t& tok0, int& n,
                                          size_t& stat0) {
  if (a.cu == nullptr) {
    tok0 = (size_t)bi * a.T;
    n = a.n;
    stat0 = (size_t)bi * a.H * a.T;
    return true;
  }
  const int c0 = a.cu[bi];
  const int c1 = a.cu[bi + 1];
  const int len = c1 - c0;
  n = (a.mode == MODE_CAUSAL) ? len : len / 2;
  tok0 = stat0 = (size_t)(c0 < 0 ? 0 : c0);
  return c0 >= 0 && len >= 0 && (long long)c1 <= a.tokens &&
         (a.mode == MODE_CAUSAL || (len & 1) == 0) && n <= a.n;
}

// Softcapping in base-2 units: for a raw score x (q.k, before the scale),
// e = 2^(x * in) = exp(2 s / cap) with s = scale * x, r = 1 / (e + 1), and
// the capped score in base 2 is out * (1 - 2 r) = cap * tanh(s / cap) * log2(e);
// its derivative with respect to s is 1 - tanh^2 = 4 r (1 - r).
struct Softcap {
  float in, out;
};
__device__ __forceinline__ Softcap softcap_consts(float scale, float cap) {
  return Softcap{scale / cap * 2.f * 1.4426950408889634f, cap * 1.4426950408889634f};
}
__device__ __forceinline__ float softcap_r(const Softcap& c, float x) {
  return __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x * c.in) + 1.f);
}
__device__ __forceinline__ float softcap_y(const Softcap& c, float r) {
  return __builtin_fmaf(-2.f * c.out, r, c.out);
}

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t s);
// q, k, v hold OCP E4M3 bytes (same layouts), with a.qd, a.kd, a.vd.
hipError_t launch_fwd_fp8(const AttnArgs& a, int D, hipStream_t s);
hipError_t launch_bwd(const AttnArgs& a, int D, hipStream_t s);
// One backward stage: 0 = dQ (also writes -delta and lse2), 1 = dK/dV
// (with the reduction of its partials when a.S > 1).
hipError_t launch_bwd_stage(const AttnArgs& a, int D, int stage, hipStream_t s);

}  // namespace bd
