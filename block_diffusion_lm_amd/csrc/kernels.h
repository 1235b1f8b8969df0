// kernels.h -- argument block and launchers of the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

struct AttnArgs {
  // inputs, bf16: q [B][T][H][D], k and v [B][T][Hkv][D]
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;     // forward output, read by the backward
  const uint16_t* dout;  // gradient of the output
  // forward outputs
  uint16_t* out;
  float* lse;            // [B][H][T], natural log
  // backward
  const float* lse_in;   // [B][H][T]
  float* ndelta;         // workspace [B][H][T]: -(dout_i . out_i)
  float* lse2;           // workspace [B][H][T]: lse * log2(e)
  uint16_t* dq;
  uint16_t* dk;   // [B][T][Hkv][D], like k
  uint16_t* dv;
  // shape
  int B, H;
  int Hkv;      // key/value heads; query head h reads key/value head h / G
  int G;        // H / Hkv, query heads per key/value head
  int S;        // dK/dV workgroups per group of query heads (divides G)
  float* part;  // S > 1: float32 partial dK then dV, each [S][B][T][Hkv][D]
  int n;        // half length (diffusion) or sequence length (causal)
  int b;        // block size (1 for causal)
  int mode;     // MODE_DIFFUSION / MODE_CAUSAL
  int T;        // tokens per sample: 2n or n
  int nhalves;  // 2 or 1
  float scale;       // multiplies q.k (may be negative)
  float scale_log2;  // scale * log2(e)
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
int dkdv_group_splits(int B, int n, int nhalves, int Hkv, int G);

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t s);
hipError_t launch_bwd(const AttnArgs& a, int D, hipStream_t s);
// One backward stage: 0 = dQ (also writes -delta and lse2), 1 = dK/dV
// (with the reduction of its partials when a.S > 1).
hipError_t launch_bwd_stage(const AttnArgs& a, int D, int stage, hipStream_t s);

}  // namespace bd
