// attn_fwd.hip -- forward pass: O = softmax(scale * Q K^T under the mask) V
// and the per-row log-sum-exp, one workgroup per 128-row query tile.
//
// FlashAttention: Exact Attention Without Materialization, sections 4.1,
// 4.2 and 5.1: a query tile streams the key/value tiles it needs through
// on-chip memory, keeps a running row maximum m, denominator l and
// unnormalised output z per row, rescales l and z by exp(m_old - m_new)
// when the maximum changes, and divides by l at the end; scores and
// probabilities never reach HBM.  Fast Diffusion Attention, "Visit only the
// visible tiles": the key tiles come from the block-diffusion enumeration
// (geometry.h) and only tiles crossing a block boundary are masked.
//
// Mapping to gfx950: 4 waves per workgroup, each owning 32 query rows.
// Scores are computed transposed, S^T = K Q^T: K (A operand) is read from
// LDS, Q (B operand) stays in registers, and each lane owns one query row,
// so the row statistics need a single exchange between the wave's halves.
// The probabilities then feed O^T += V^T P^T as the B operand directly from
// the score registers; V^T comes from the natural V tile through
// transposing LDS reads.  K/V tiles are double-buffered in LDS and filled
// by buffer loads that write LDS directly, issued one tile ahead.  Every
// wave classifies each 32-key block of a tile against its own rows and
// skips blocks it cannot see (the per-wave analogue of computing the noisy
// diagonal at reduced width).
//
// The running maximum is raised lazily: z and l are rescaled only when a
// row's maximum grows by more than 2^8 (in base-2 units), otherwise the old
// maximum stays the reference and probabilities up to 2^8 are accumulated.
// Because z and l always share one reference, the result is the same
// function (section 4.2's recurrence holds for any common reference); this
// removes the per-tile rescale of z in the common case.
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
  using Tile = DirectTile<BN, D, NT>;
  static constexpr int BUF = 2 * Tile::ELEMS;  // K then V
};

constexpr float kRescaleThreshold = 8.0f;  // log2 units

__device__ __forceinline__ int half_offset(const AttnArgs& a, int half) {
  return (a.mode == MODE_DIFFUSION && half == CLEAN) ? a.n : 0;
}

// What a query-stationary wave needs about one key half: the visible
// intervals of its first and last rows (block classification), of this
// lane's row (element mask), and the K / V resources of that half.
struct RowSeg {
  int lo_f, hi_f, lo_l, hi_l, lo_p, hi_p;
  rsrc_t rk, rv;
};

template <int D>
__device__ __forceinline__ RowSeg make_row_seg(const AttnArgs& a, const Geom& g, int qh, int kh, int pw0,
                                               int pw1, int p, size_t sample0, size_t rs, int hh,
                                               uint32_t half_bytes) {
  RowSeg s;
  row_interval(g, qh, kh, pw0, s.lo_f, s.hi_f);
  row_interval(g, qh, kh, max(pw1 - 1, pw0), s.lo_l, s.hi_l);
  row_interval(g, qh, kh, p, s.lo_p, s.hi_p);
  const size_t base = (sample0 + half_offset(a, kh)) * rs + (size_t)hh * D;
  s.rk = make_rsrc(a.k + base, half_bytes);
  s.rv = make_rsrc(a.v + base, half_bytes);
  return s;
}

template <int D, int BN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnArgs a, int qtiles) {
  using C = FwdCfg<D, BN>;
  using Tile = typename C::Tile;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * C::BUF];

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
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const uint32_t half_bytes = (uint32_t)a.n * row_bytes;

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, a.n);
  const bool wave_active = pw0 < a.n;
  const int p = pw0 + l32;

  // Q^T operand: lane (row p, half h2) holds Q[p][16s + 8h2 .. +7]; rows past
  // the half read as zero.  A negative scale is folded into Q (exact in
  // bf16) so that the softmax below always works with a positive factor.
  bf16x8 qf[C::KS];
  {
    const rsrc_t rq = make_rsrc(a.q + (sample0 + qoff) * rs + (size_t)hh * D, half_bytes);
    const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 v = buf_ld16(rq, (uint32_t)p * row_bytes + (uint32_t)(16 * s + 8 * h2) * 2u, 0);
      v ^= flip;
      qf[s] = as_bf16x8(v);
    }
  }
  const float cs = fabsf(a.scale) * kLog2e;

  const Segments seg = fwd_segments(g, a.mode, qh, qt, C::BM, BN);
  const int n0 = seg.count > 0 ? seg.end0 - seg.begin0 : 0;
  const int ntiles = seg.tiles();

  // Per segment: the wave's first/last row intervals (block classification),
  // this lane's interval (element mask) and the K/V resources.
  const RowSeg s0 = make_row_seg<D>(a, g, qh, seg.half0, pw0, pw1, p, sample0, rs, hh, half_bytes);
  const RowSeg s1 = make_row_seg<D>(a, g, qh, seg.half1, pw0, pw1, p, sample0, rs, hh, half_bytes);

  auto issue_tile = [&](int i, int buf) {
    const bool second = i >= n0;
    const int kt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
    uint16_t* dst = smem + buf * C::BUF;
    Tile::load(second ? s1.rk : s0.rk, row_bytes, kt * BN, dst, tid);
    Tile::load(second ? s1.rv : s0.rv, row_bytes, kt * BN, dst + Tile::ELEMS, tid);
  };

  floatx16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = zero16();
  float m_run = -INFINITY;  // running maximum, base-2 units, scale applied
  float l_run = 0.f;        // this lane's share of the denominator

  if (ntiles > 0) issue_tile(0, 0);
  wait_vmem();
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const bool more = i + 1 < ntiles;
    if (more) issue_tile(i + 1, (i + 1) & 1);
    const uint16_t* Ks = smem + (i & 1) * C::BUF;
    const uint16_t* Vs = Ks + Tile::ELEMS;

    if (wave_active) {
      const bool second = i >= n0;
      const RowSeg& sg = second ? s1 : s0;
      const int k0 = (second ? seg.begin1 + (i - n0) : seg.begin0 + i) * BN;
      const int lf = sg.lo_f, hf = sg.hi_f, ll = sg.lo_l, hl = sg.hi_l;
      const int lo = sg.lo_p, hi = sg.hi_p;
      int cls[C::KB];
      floatx16 sc[C::KB];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int c0 = k0 + 32 * kb;
        cls[kb] = (c0 >= hl || c0 + 32 <= lf) ? TILE_SKIP
                  : (ll <= c0 && c0 + 32 <= hf) ? TILE_FULL
                                                : TILE_PARTIAL;
        if (cls[kb] == TILE_SKIP) continue;
        floatx16 acc = zero16();
#pragma unroll
        for (int s = 0; s < C::KS; ++s) acc = mfma32(lds_row8<D>(Ks, 32 * kb + l32, 2 * s + h2), qf[s], acc);
        if (cls[kb] == TILE_PARTIAL) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = c0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            acc[r] = (key >= lo && key < hi) ? acc[r] : -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, acc[r]);
        sc[kb] = acc;
      }
      // raw scores -> base-2 units with the positive factor cs
      const float m_tile = halves_max(mt) * cs;
      const float m_cand = fmaxf(m_run, m_tile);
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleThreshold)) {
        // 0 when m_run is -inf; 1 for rows whose maximum did not move
        // (including rows that have seen no key yet, where both are -inf)
        const float alpha = (m_cand > m_run) ? fast_exp2(m_run - m_cand) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_cand;
      }
      const float nbase = (m_run == -INFINITY) ? 0.f : -m_run;

#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        if (cls[kb] == TILE_SKIP) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(__builtin_fmaf(sc[kb][r], cs, nbase));
          sc[kb][r] = pr;
          l_run += pr;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = pack_bf16x8(sc[kb], 8 * ks);
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            o[db] = mfma32(lds_trA<D>(Vs, 32 * kb + 16 * ks, 32 * db, lane), pb, o[db]);
        }
      }
    }

    wait_vmem();
    __syncthreads();
  }

  // Epilogue: O = z / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = halves_sum(l_run);
  if (wave_active && p < a.n) {
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
