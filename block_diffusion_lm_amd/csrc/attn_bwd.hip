// attn_bwd.hip -- backward pass, split in three kernels:
//
//   preprocess : delta_i = dO_i . O_i (float32), the row term of dS;
//   dkdv       : one workgroup per 128-key tile; it walks the query tiles
//                that see its keys and accumulates dV = P^T dO and
//                dK = scale * dS^T Q in registers;
//   dq         : one workgroup per 128-row query tile; it walks the key
//                tiles its rows see and accumulates dQ = scale * dS K.
//
// FlashAttention: Exact Attention Without Materialization, section 4.5:
// the probabilities are recomputed on chip from Q, K and the saved
// log-sum-exp (P = exp(scale * q.k - LSE)) rather than stored.  With
// dP = dO V^T, dS = P * (dP - delta).  Fast Diffusion Attention, "Visit only
// the visible tiles": each key tile visits exactly the query tiles that see
// it (geometry.h, bwd_segments), each query tile exactly the key tiles it
// sees.  Neither kernel uses atomics, so the result is deterministic.
//
// Mapping to gfx950 (MFMA layouts in common.h):
//  dkdv: each wave owns 32 keys, holding K and V as B operands in registers
//    for the whole walk.  S = Q K^T and dP = dO V^T come out with one key
//    per lane and query rows in registers; read with k = query row they are
//    directly the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//    operands (dO^T, Q^T) come from transposed LDS copies.  Q and dO tiles
//    are double-buffered in LDS in natural and transposed layouts.
//  dq: each wave owns 32 query rows, holding Q and dO as B operands.
//    S^T = K Q^T and dP^T = V dO^T give one query per lane (so LSE and delta
//    are per-lane scalars); dQ^T += K^T dS^T takes K^T from a transposed LDS
//    copy of the key tile.
#include "common.h"
#include "geometry.h"
#include "kernels.h"
#include "tile_io.h"

namespace bd {

__device__ __forceinline__ int half_off(const AttnArgs& a, int half) {
  return (a.mode == MODE_DIFFUSION && half == CLEAN) ? a.n : 0;
}

// ---------------------------------------------------------------------------
// delta_i = sum_d dO[i][d] * O[i][d]; one 16-byte chunk per lane, rows of
// D / 8 lanes reduced with cross-lane shuffles.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(AttnArgs a, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = ld16(a.o + row * D + c * 8);
    const u32x4 gv = ld16(a.dout + row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __builtin_bit_cast(float, ov[w] << 16) * __builtin_bit_cast(float, gv[w] << 16);
      acc += __builtin_bit_cast(float, ov[w] & 0xffff0000u) * __builtin_bit_cast(float, gv[w] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && c == 0) {
    // row = (b * T + t) * H + h  ->  delta[(b * H + h) * T + t]
    const long long h = row % a.H;
    const long long bt = row / a.H;
    const long long t = bt % a.T;
    const long long b = bt / a.T;
    a.delta[(b * a.H + h) * a.T + t] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary.
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BKV = 32 * NW;  // keys per workgroup
  static constexpr int BQ = 64;        // query rows per streamed tile
  static constexpr int QB = BQ / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  using QL = TileLoader<BQ, D, NT>;
  static constexpr int QN_OFF = 0;
  static constexpr int QT_OFF = QN_OFF + QL::NAT_ELEMS;
  static constexpr int DN_OFF = QT_OFF + QL::T_ELEMS;
  static constexpr int DT_OFF = DN_OFF + QL::NAT_ELEMS;
  static constexpr int BUF16 = DT_OFF + QL::T_ELEMS;  // bf16 elements per buffer
  static constexpr int FBUF = 2 * BQ;                 // floats per buffer: lse2, delta
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(AttnArgs a, int ktiles) {
  using C = DkdvCfg<D>;
  using QL = typename C::QL;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF16];
  __shared__ __attribute__((aligned(16))) float fsm[2 * C::FBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // Clean key tiles in increasing order (the earliest keys are seen by the
  // most rows), then the noisy key tiles, which only their own blocks see.
  const int BH = a.B * a.H;
  const int bid = blockIdx.x;
  int kh, kt, bh;
  if (bid < ktiles * BH) {
    kh = CLEAN;
    kt = bid / BH;
    bh = bid % BH;
  } else {
    kh = NOISY;
    kt = (bid - ktiles * BH) / BH;
    bh = (bid - ktiles * BH) % BH;
  }
  const int bi = bh / a.H;
  const int hh = bh % a.H;
  const Geom g{a.n, a.b};
  const size_t rs = (size_t)a.H * D;
  const size_t sample0 = (size_t)bi * a.T;
  const int koff = half_off(a, kh);

  const int k0 = kt * C::BKV;
  const int kw0 = k0 + 32 * w;          // this wave's first key
  const bool wave_active = kw0 < a.n;
  const int key = kw0 + l32;            // this lane's key
  const bool key_ok = key < a.n;

  // K and V as B operands: lane (key, h2) holds row[16s + 8h2 .. +7].
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const size_t off = (sample0 + koff + key) * rs + (size_t)hh * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      kf[s] = as_bf16x8(key_ok ? ld16(a.k + off + 16 * s + 8 * h2) : zero_u32x4());
      vf[s] = as_bf16x8(key_ok ? ld16(a.v + off + 16 * s + 8 * h2) : zero_u32x4());
    }
  }

  const Segments seg = bwd_segments(g, a.mode, kh, kt, C::BQ, C::BKV);
  const int n0 = seg.count > 0 ? seg.end[0] - seg.begin[0] : 0;
  const int ntiles = n0 + (seg.count > 1 ? seg.end[1] - seg.begin[1] : 0);
  auto tile_at = [&](int i, int& qh, int& qt) {
    if (i < n0) {
      qh = seg.half[0];
      qt = seg.begin[0] + i;
    } else {
      qh = seg.half[1];
      qt = seg.begin[1] + (i - n0);
    }
  };
  auto row_base = [&](const uint16_t* t, int qh) {
    return t + (sample0 + half_off(a, qh)) * rs + (size_t)hh * D;
  };
  const size_t stat_base = ((size_t)bi * a.H + hh) * a.T;

  floatx16 dk[C::DB], dv[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  QL qload, dload;
  float st_l = 0.f, st_d = 0.f;  // this thread's lse2 / delta entry (threads < BQ)
  auto load_tile = [&](int i) {
    int qh, qt;
    tile_at(i, qh, qt);
    qload.load(row_base(a.q, qh), rs, qt * C::BQ, a.n, tid);
    dload.load(row_base(a.dout, qh), rs, qt * C::BQ, a.n, tid);
    if (tid < C::BQ) {
      const int r = qt * C::BQ + tid;
      const bool ok = r < a.n;
      const size_t si = stat_base + half_off(a, qh) + r;
      // rows past the half get LSE = +inf, so their probabilities are 0
      st_l = ok ? a.lse_in[si] * kLog2e : INFINITY;
      st_d = ok ? a.delta[si] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* b16 = smem + buf * C::BUF16;
    qload.store_nat(b16 + C::QN_OFF, tid);
    qload.store_t(b16 + C::QT_OFF, tid);
    dload.store_nat(b16 + C::DN_OFF, tid);
    dload.store_t(b16 + C::DT_OFF, tid);
    if (tid < C::BQ) {
      fsm[buf * C::FBUF + tid] = st_l;
      fsm[buf * C::FBUF + C::BQ + tid] = st_d;
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    int qh, qt;
    tile_at(i, qh, qt);
    const bool more = i + 1 < ntiles;
    if (more) load_tile(i + 1);
    const int buf = i & 1;
    const uint16_t* Qs = smem + buf * C::BUF16 + C::QN_OFF;
    const uint16_t* Qt = smem + buf * C::BUF16 + C::QT_OFF;
    const uint16_t* Ds = smem + buf * C::BUF16 + C::DN_OFF;
    const uint16_t* Dt = smem + buf * C::BUF16 + C::DT_OFF;
    const float* Ls = fsm + buf * C::FBUF;
    const float* Dl = Ls + C::BQ;

    if (wave_active) {
      int clo, chi;  // rows of half qh that see this lane's key
      col_interval(g, qh, kh, key, clo, chi);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const int r0 = qt * C::BQ + 32 * qb;
        if (r0 >= a.n) continue;
        const int r1 = min(r0 + 32, a.n);
        const int cls = classify(g, qh, kh, r0, r1, kw0, kw0 + 32);
        if (cls == TILE_SKIP) continue;

        floatx16 sp = zero16(), dp = zero16();
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          sp = mfma32(lds_nat<D>(Qs, 32 * qb + l32, 2 * s + h2), kf[s], sp);
          dp = mfma32(lds_nat<D>(Ds, 32 * qb + l32, 2 * s + h2), vf[s], dp);
        }
        // P = exp2(S * scale * log2 e - LSE * log2 e); dS = P * (dP - delta)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int rl = 32 * qb + 8 * gq + 4 * h2;  // tile-local row of register 4gq
          const float4 l4 = *reinterpret_cast<const float4*>(Ls + rl);
          const float4 d4 = *reinterpret_cast<const float4*>(Dl + rl);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * gq + j;
            float pr = fast_exp2(sp[r] * a.scale_log2 - lv[j]);
            if (cls == TILE_PARTIAL) {
              const int row = qt * C::BQ + rl + j;
              if (row < clo || row >= chi) pr = 0.f;
            }
            sp[r] = pr;
            dp[r] = pr * (dp[r] - dl[j]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = pack_bf16x8(sp, 8 * ks);
          const bf16x8 sb = pack_bf16x8(dp, 8 * ks);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int toff = (32 * db + l32) * QL::T_STRIDE + 32 * qb + 16 * ks + 8 * h2;
            dv[db] = mfma32(lds_vec(Dt + toff), pb, dv[db]);
            dk[db] = mfma32(lds_vec(Qt + toff), sb, dk[db]);
          }
        }
      }
    }

    if (more) store_tile((i + 1) & 1);
    __syncthreads();
  }

  // dK^T / dV^T: lane = key, register r of block db = dimension
  // 32db + 8(r/4) + 4h2 + r%4.
  if (wave_active && key_ok) {
    const size_t off = (sample0 + koff + key) * rs + (size_t)hh * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * h2;
        u32x2 kv = {pack2_bf16(dk[db][4 * gq] * a.scale, dk[db][4 * gq + 1] * a.scale),
                    pack2_bf16(dk[db][4 * gq + 2] * a.scale, dk[db][4 * gq + 3] * a.scale)};
        u32x2 vv = {pack2_bf16(dv[db][4 * gq], dv[db][4 * gq + 1]),
                    pack2_bf16(dv[db][4 * gq + 2], dv[db][4 * gq + 3])};
        *reinterpret_cast<u32x2*>(a.dk + off + d) = kv;
        *reinterpret_cast<u32x2*>(a.dv + off + d) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary.
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int KB = BN / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  using KL = TileLoader<BN, D, NT>;
  static constexpr int KN_OFF = 0;
  static constexpr int KT_OFF = KN_OFF + KL::NAT_ELEMS;
  static constexpr int VN_OFF = KT_OFF + KL::T_ELEMS;
  static constexpr int BUF = VN_OFF + KL::NAT_ELEMS;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(AttnArgs a, int qtiles) {
  using C = DqCfg<D>;
  using KL = typename C::KL;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  const int BH = a.B * a.H;
  const int R = a.nhalves * BH;
  const int bid = blockIdx.x;
  const int qt = qtiles - 1 - bid / R;
  const int rr = bid % R;
  const int half_idx = rr / BH;
  const int bh = rr % BH;
  const int bi = bh / a.H;
  const int hh = bh % a.H;
  const int qh = (a.mode == MODE_CAUSAL) ? CLEAN : half_idx;
  const Geom g{a.n, a.b};
  const size_t rs = (size_t)a.H * D;
  const size_t sample0 = (size_t)bi * a.T;
  const int qoff = half_off(a, qh);

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, a.n);
  const bool wave_active = pw0 < a.n;
  const int p = pw0 + l32;
  const bool row_ok = p < a.n;

  bf16x8 qf[C::KS], gf[C::KS];
  {
    const size_t off = (sample0 + qoff + p) * rs + (size_t)hh * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      qf[s] = as_bf16x8(row_ok ? ld16(a.q + off + 16 * s + 8 * h2) : zero_u32x4());
      gf[s] = as_bf16x8(row_ok ? ld16(a.dout + off + 16 * s + 8 * h2) : zero_u32x4());
    }
  }
  const size_t si = ((size_t)bi * a.H + hh) * a.T + qoff + p;
  const float lse2 = row_ok ? a.lse_in[si] * kLog2e : INFINITY;
  const float dlt = row_ok ? a.delta[si] : 0.f;

  const Segments seg = fwd_segments(g, a.mode, qh, qt, C::BM, BN);
  const int n0 = seg.count > 0 ? seg.end[0] - seg.begin[0] : 0;
  const int ntiles = n0 + (seg.count > 1 ? seg.end[1] - seg.begin[1] : 0);
  auto tile_at = [&](int i, int& kh, int& kt) {
    if (i < n0) {
      kh = seg.half[0];
      kt = seg.begin[0] + i;
    } else {
      kh = seg.half[1];
      kt = seg.begin[1] + (i - n0);
    }
  };
  auto kv_base = [&](const uint16_t* t, int kh) {
    return t + (sample0 + half_off(a, kh)) * rs + (size_t)hh * D;
  };

  floatx16 dq[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) dq[i] = zero16();

  KL kload, vload;
  if (ntiles > 0) {
    int kh, kt;
    tile_at(0, kh, kt);
    kload.load(kv_base(a.k, kh), rs, kt * BN, a.n, tid);
    vload.load(kv_base(a.v, kh), rs, kt * BN, a.n, tid);
    kload.store_nat(smem + C::KN_OFF, tid);
    kload.store_t(smem + C::KT_OFF, tid);
    vload.store_nat(smem + C::VN_OFF, tid);
  }
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    int kh, kt;
    tile_at(i, kh, kt);
    const bool more = i + 1 < ntiles;
    if (more) {
      int kh2, kt2;
      tile_at(i + 1, kh2, kt2);
      kload.load(kv_base(a.k, kh2), rs, kt2 * BN, a.n, tid);
      vload.load(kv_base(a.v, kh2), rs, kt2 * BN, a.n, tid);
    }
    const uint16_t* Ks = smem + (i & 1) * C::BUF + C::KN_OFF;
    const uint16_t* Kt = smem + (i & 1) * C::BUF + C::KT_OFF;
    const uint16_t* Vs = smem + (i & 1) * C::BUF + C::VN_OFF;

    if (wave_active) {
      const int k0 = kt * BN;
      int lo, hi;
      row_interval(g, qh, kh, p, lo, hi);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int c0 = k0 + 32 * kb;
        if (c0 >= a.n) continue;
        const int cls = classify(g, qh, kh, pw0, pw1, c0, c0 + 32);
        if (cls == TILE_SKIP) continue;
        floatx16 sp = zero16(), dp = zero16();
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          sp = mfma32(lds_nat<D>(Ks, 32 * kb + l32, 2 * s + h2), qf[s], sp);
          dp = mfma32(lds_nat<D>(Vs, 32 * kb + l32, 2 * s + h2), gf[s], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(sp[r] * a.scale_log2 - lse2);
          if (cls == TILE_PARTIAL) {
            const int kk = c0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (kk < lo || kk >= hi) pr = 0.f;
          }
          dp[r] = pr * (dp[r] - dlt);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 sb = pack_bf16x8(dp, 8 * ks);
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            dq[db] = mfma32(lds_vec(Kt + (32 * db + l32) * KL::T_STRIDE + 32 * kb + 16 * ks + 8 * h2), sb, dq[db]);
        }
      }
    }

    if (more) {
      uint16_t* nb = smem + ((i + 1) & 1) * C::BUF;
      kload.store_nat(nb + C::KN_OFF, tid);
      kload.store_t(nb + C::KT_OFF, tid);
      vload.store_nat(nb + C::VN_OFF, tid);
    }
    __syncthreads();
  }

  if (wave_active && row_ok) {
    uint16_t* qrow = a.dq + (sample0 + qoff + p) * rs + (size_t)hh * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * h2;
        u32x2 pk = {pack2_bf16(dq[db][4 * gq] * a.scale, dq[db][4 * gq + 1] * a.scale),
                    pack2_bf16(dq[db][4 * gq + 2] * a.scale, dq[db][4 * gq + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(qrow + d) = pk;
      }
  }
}

template <int D>
static hipError_t launch_stage_t(const AttnArgs& a, int stage, hipStream_t s) {
  if (stage == 0) {
    const long long rows = (long long)a.B * a.T * a.H;
    constexpr int rows_per_block = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(256), 0, s, a, rows);
  } else if (stage == 1) {
    using KC = DkdvCfg<D>;
    const int ktiles = (a.n + KC::BKV - 1) / KC::BKV;
    const long long kblocks = (long long)ktiles * a.nhalves * a.B * a.H;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)kblocks), dim3(KC::NT), 0, s, a, ktiles);
  } else {
    using QC = DqCfg<D>;
    const int qtiles = (a.n + QC::BM - 1) / QC::BM;
    const long long qblocks = (long long)qtiles * a.nhalves * a.B * a.H;
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)qblocks), dim3(QC::NT), 0, s, a, qtiles);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_stage(const AttnArgs& a, int D, int stage, hipStream_t s) {
  return D == 64 ? launch_stage_t<64>(a, stage, s) : launch_stage_t<128>(a, stage, s);
}

hipError_t launch_bwd(const AttnArgs& a, int D, hipStream_t s) {
  for (int stage = 0; stage < 3; ++stage) {
    hipError_t e = launch_bwd_stage(a, D, stage, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bd
