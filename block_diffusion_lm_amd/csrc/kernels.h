// kernels.h -- argument block and launchers of the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

struct AttnArgs {
  // inputs, bf16 [B][T][H][D]
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
  uint16_t* dk;
  uint16_t* dv;
  // shape
  int B, H;
  int n;        // half length (diffusion) or sequence length (causal)
  int b;        // block size (1 for causal)
  int mode;     // MODE_DIFFUSION / MODE_CAUSAL
  int T;        // tokens per sample: 2n or n
  int nhalves;  // 2 or 1
  float scale;       // multiplies q.k (may be negative)
  float scale_log2;  // scale * log2(e)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t s);
hipError_t launch_bwd(const AttnArgs& a, int D, hipStream_t s);
// One backward kernel: 0 = dQ (also writes -delta and lse2), 1 = dK/dV.
hipError_t launch_bwd_stage(const AttnArgs& a, int D, int stage, hipStream_t s);

}  // namespace bd
