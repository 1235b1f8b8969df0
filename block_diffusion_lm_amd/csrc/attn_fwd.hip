// attn_fwd.hip -- forward pass: O = softmax(scale * Q K^T under the mask) V
// and the per-row log-sum-exp, one workgroup per 128-row query tile.
//
// FlashAttention: Exact Attention Without Materialization, sections 4.1,
// 4.2 and 5.1: a query tile streams the key/value tiles it needs through
// on-chip memory, keeps a running row maximum m, denominator l and
// unnormalised output z per row, rescales them by exp(m_old - m_new) when
// the maximum grows and divides by l at the end; scores and probabilities
// never reach HBM.  Fast Diffusion Attention, "Visit only the visible
// tiles": the key tiles come from the block-diffusion enumeration
// (geometry.h) and only tiles crossing a block boundary are masked.
//
// Mapping to gfx950: 4 waves per workgroup, each owning 32 query rows.
// Scores are computed transposed, S^T = K Q^T (K is the MFMA A operand
// read from LDS, Q the B operand kept in registers), so that a lane owns
// one query row and the row statistics need a single cross-half exchange;
// the probabilities then feed O^T += V^T P^T as the B operand straight from
// the score registers, with V^T read from a transposed LDS copy.  K/V tiles
// are double-buffered in LDS with the next tile's global loads in flight
// during the current tile's math (one barrier per tile).  Inside a tile,
// every wave classifies each 32-key block against its own rows and skips
// blocks it cannot see (the per-wave analogue of computing the noisy
// diagonal at reduced width).
#include "common.h"
#include "geometry.h"
#include "kernels.h"
#include "tile_io.h"

namespace bd {

template <int D, int BN>
struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  static constexpr int DB = D / 32;   // 32-wide column blocks of the head dimension
  static constexpr int KB = BN / 32;  // 32-key blocks per key tile
  using KL = TileLoader<BN, D, NT>;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KL::NAT_ELEMS;
  static constexpr int BUF = KL::NAT_ELEMS + KL::T_ELEMS;  // elements per buffer
};

__device__ __forceinline__ int half_offset(const AttnArgs& a, int half) {
  return (a.mode == MODE_DIFFUSION && half == CLEAN) ? a.n : 0;
}

template <int D, int BN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnArgs a, int qtiles) {
  using C = FwdCfg<D, BN>;
  using KL = typename C::KL;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // Heaviest query tiles first; within one tile index, both halves of a
  // (sample, head) sit at the same residue modulo the XCD count when B*H is
  // a multiple of 8, so they share an L2.
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
  const int qoff = half_offset(a, qh);

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, a.n);
  const bool wave_active = pw0 < a.n;
  const int p = pw0 + l32;
  const bool row_ok = p < a.n;

  // Q^T operand: lane (row p, half h2) holds Q[p][16s + 8h2 .. +7].
  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = a.q + (sample0 + qoff + p) * rs + (size_t)hh * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qf[s] = as_bf16x8(row_ok ? ld16(qrow + 16 * s + 8 * h2) : zero_u32x4());
  }

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
    return t + (sample0 + half_offset(a, kh)) * rs + (size_t)hh * D;
  };

  floatx16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  KL kload, vload;
  if (ntiles > 0) {
    int kh, kt;
    tile_at(0, kh, kt);
    kload.load(kv_base(a.k, kh), rs, kt * BN, a.n, tid);
    vload.load(kv_base(a.v, kh), rs, kt * BN, a.n, tid);
    kload.store_nat(smem + C::K_OFF, tid);
    vload.store_t(smem + C::V_OFF, tid);
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
    const uint16_t* Ks = smem + (i & 1) * C::BUF + C::K_OFF;
    const uint16_t* Vt = smem + (i & 1) * C::BUF + C::V_OFF;

    if (wave_active) {
      const int k0 = kt * BN;
      int lo, hi;
      row_interval(g, qh, kh, p, lo, hi);
      int cls[C::KB];
      floatx16 sc[C::KB];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int c0 = k0 + 32 * kb;
        cls[kb] = (c0 < a.n) ? classify(g, qh, kh, pw0, pw1, c0, c0 + 32) : TILE_SKIP;
        if (cls[kb] == TILE_SKIP) continue;
        floatx16 acc = zero16();
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
          acc = mfma32(lds_nat<D>(Ks, 32 * kb + l32, 2 * s + h2), qf[s], acc);
        if (cls[kb] == TILE_PARTIAL) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = c0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            float x = acc[r] * a.scale_log2;
            acc[r] = (key >= lo && key < hi) ? x : -INFINITY;
            mt = fmaxf(mt, acc[r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[r] *= a.scale_log2;
            mt = fmaxf(mt, acc[r]);
          }
        }
        sc[kb] = acc;
      }
      mt = halves_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - base);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;

#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        if (cls[kb] == TILE_SKIP) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(sc[kb][r] - base);
          sc[kb][r] = pr;
          l_run += pr;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = pack_bf16x8(sc[kb], 8 * ks);
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            o[db] = mfma32(lds_vec(Vt + (32 * db + l32) * KL::T_STRIDE + 32 * kb + 16 * ks + 8 * h2), pb, o[db]);
        }
      }
    }

    if (more) {
      uint16_t* nb = smem + ((i + 1) & 1) * C::BUF;
      kload.store_nat(nb + C::K_OFF, tid);
      vload.store_t(nb + C::V_OFF, tid);
    }
    __syncthreads();
  }

  // Epilogue: O = z / l, LSE = (m + log2 l) * ln 2 (m is in log2 units).
  const float l_tot = halves_sum(l_run);
  if (wave_active && row_ok) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.out + (sample0 + qoff + p) * rs + (size_t)hh * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * h2;
        u32x2 pk = {pack2_bf16(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                    pack2_bf16(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
    if (h2 == 0)
      a.lse[((size_t)bi * a.H + hh) * a.T + qoff + p] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, int BN>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t s) {
  using C = FwdCfg<D, BN>;
  const int qtiles = (a.n + C::BM - 1) / C::BM;
  const long long blocks = (long long)qtiles * a.nhalves * a.B * a.H;
  hipLaunchKernelGGL((fwd_kernel<D, BN>), dim3((unsigned)blocks), dim3(C::NT), 0, s, a, qtiles);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t s) {
  if (D == 64) return launch_fwd_t<64, 64>(a, s);
  return launch_fwd_t<128, 64>(a, s);
}

}  // namespace bd
