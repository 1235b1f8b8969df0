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

#include <type_traits>

namespace bd {

template <int D, int BN, int NW_ = 4, int NBUF_ = 2>
struct FwdCfg {
  static constexpr int NW = NW_;      // waves per workgroup (32 query rows each)
  static constexpr int NBUF = NBUF_;  // depth of the K/V ring in LDS
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  static constexpr int DB = D / 32;   // 32-wide column blocks of the head dimension
  static constexpr int KB = BN / 32;  // 32-key blocks per key tile
  using Tile = DirectTile<BN, D, NT>;
  static_assert(Tile::SLOTS % NT == 0, "the counted tile waits assume PER loads per tile in every wave");
  static constexpr int BUF = 2 * Tile::ELEMS;  // K then V
};

constexpr float kRescaleThreshold = 8.0f;  // log2 units

// Token offset of a half inside its sample (n: the sample's half length).
__device__ __forceinline__ int half_offset(const AttnArgs& a, int half, int n) {
  return (a.mode == MODE_DIFFUSION && half == CLEAN) ? n : 0;
}

// SC: softcapping on (the scores are capped before the mask and the
// maximum, and kept in base-2 units).
template <int D, int BN, int NW, int NBUF, bool SC>
// D = 128: 32-key K / V tiles (32 KiB of LDS) and at most 168 registers,
// three workgroups per CU.  D = 96: 64-key tiles (48 KiB) and at most 168
// registers, three workgroups per CU.  D = 192 and 256: 32-key tiles, two
// workgroups per CU (Q and O take most of half a register file).  D = 64: at
// most 128 registers, four workgroups per CU.
__global__ __launch_bounds__(64 * NW, (D == 64 ? 4 : ((D == 128 && BN == 32) || (D == 96 && NW == 4)) ? 3 : (NW == 4 && (D < 192 || BN == 32) ? 2 : 1))) void fwd_kernel(AttnArgs a, int qtiles) {
  using C = FwdCfg<D, BN, NW, NBUF>;
  using Tile = typename C::Tile;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NBUF * C::BUF];
  const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_byte_addr(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // Heaviest query tiles first; within one tile index, both halves of a
  // (sample, head) sit at the same residue modulo the XCD count when B*H is
  // a multiple of 8, so they share an L2 (and so do the query heads of one
  // key/value head, see query_head).
  const int BH = a.B * a.H;
  const int R = a.nhalves * BH;
  const int bid = blockIdx.x;
  const int qt = qtiles - 1 - bid / R;
  const int rr = bid % R;
  const int half_idx = rr / BH;
  int bi, hh, hk;
  query_head(a, rr % BH, bi, hh, hk);
  const int qh = (a.mode == MODE_CAUSAL) ? CLEAN : half_idx;
  size_t sample0, stat0;
  int n;
  // packed samples shorter than the longest leave their last tiles empty
  if (!sample_of(a, bi, sample0, n, stat0) || qt * C::BM >= n) return;
  const Geom g{n, a.b};

  // Q / O rows hold H heads, K / V rows Hkv heads.
  const size_t rs = (size_t)a.H * D;
  const size_t rs_kv = (size_t)a.Hkv * D;
  const int qoff = half_offset(a, qh, n);
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const uint32_t half_bytes = (uint32_t)n * row_bytes;
  const uint32_t kv_row_bytes = (uint32_t)rs_kv * 2u;
  const uint32_t kv_half_bytes = (uint32_t)n * kv_row_bytes;

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, n);
  const bool wave_active = pw0 < n;
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
#pragma unroll
    for (int s = 0; s < C::KS; ++s) settle(qf[s]);
  }
  // Without softcapping the raw scores are scaled by cs when used; with it
  // they are first turned into capped base-2 scores (factor 1 afterwards).
  // Q carries the sign of the scale, so the raw scores are scaled by |scale|.
  const Softcap capc = SC ? softcap_consts(fabsf(a.scale), a.softcap) : Softcap{0.f, 0.f};
  const float cs = SC ? 1.f : fabsf(a.scale) * kLog2e;

  const Segments seg = fwd_segments(g, a.mode, qh, qt, C::BM, BN);
  const int n0 = seg.count > 0 ? seg.end0 - seg.begin0 : 0;
  const int ntiles = seg.tiles();

  // Per segment (key half): the visible intervals of the wave's first and
  // last rows (block classification), of this lane's row (element mask),
  // and row 0 of K / V in that half.  Kept as separate scalars and picked
  // with selects: grouping them in a struct lets the compiler select
  // between the structs' addresses, which puts both in scratch memory.
  int lo_f0, hi_f0, lo_l0, hi_l0, lo_p0, hi_p0, lo_f1, hi_f1, lo_l1, hi_l1, lo_p1, hi_p1;
  row_interval(g, qh, seg.half0, pw0, lo_f0, hi_f0);
  row_interval(g, qh, seg.half0, max(pw1 - 1, pw0), lo_l0, hi_l0);
  row_interval(g, qh, seg.half0, p, lo_p0, hi_p0);
  row_interval(g, qh, seg.half1, pw0, lo_f1, hi_f1);
  row_interval(g, qh, seg.half1, max(pw1 - 1, pw0), lo_l1, hi_l1);
  row_interval(g, qh, seg.half1, p, lo_p1, hi_p1);
  // The blocks of the wave's first and last rows and of this lane's row.
  // At D >= 192 and with 32-key tiles the intervals of a tile's half are
  // derived from these per tile: selected from the two halves' copies, they
  // ended up read through a table of addresses in scratch memory.
  const int bs_f = g.bstart(pw0), be_f = g.bend(pw0);
  const int bs_l = g.bstart(max(pw1 - 1, pw0)), be_l = g.bend(max(pw1 - 1, pw0));
  const int bs_p = g.bstart(p), be_p = g.bend(p);
  const size_t kvb0 = (sample0 + half_offset(a, seg.half0, n)) * rs_kv + (size_t)hk * D;
  const size_t kvb1 = (sample0 + half_offset(a, seg.half1, n)) * rs_kv + (size_t)hk * D;

  auto issue_tile = [&](int i, int buf) __attribute__((always_inline)) {
    const bool second = i >= n0;
    const int kt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
    const size_t kvb = second ? kvb1 : kvb0;
    const uint32_t dst = sbase + (uint32_t)(buf * C::BUF) * 2u;
    Tile::load(make_rsrc(a.k + kvb, kv_half_bytes), kv_row_bytes, kt * BN, dst, tid);
    Tile::load(make_rsrc(a.v + kvb, kv_half_bytes), kv_row_bytes, kt * BN, dst + Tile::ELEMS * 2u, tid);
  };

  floatx16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = zero16();
  float m_run = -INFINITY;  // running maximum, base-2 units, scale applied
  float l_run = 0.f;        // this lane's share of the denominator (float32 P: the LSE)
  float lr_run = 0.f;       // the same sum over P as rounded to bf16 for P.V (normalises O)

  // Per-lane parts of the LDS addresses, fixed for the whole walk: one
  // entry per chunk position within the swizzle's span (k-step s reads
  // chunk 2s + h2, column block db chunks 4db ..); the span-multiples are
  // compile-time offsets.
  constexpr int KP = swz_span<D>() / 2 < C::KS ? swz_span<D>() / 2 : C::KS;
  constexpr int DP = swz_span<D>() / 4 < C::DB ? swz_span<D>() / 4 : C::DB;
  int koff_[KP];
#pragma unroll
  for (int s = 0; s < KP; ++s) koff_[s] = row8_lane_off<D>(lane, 2 * s);
  int voff_[DP][2];
#pragma unroll
  for (int db = 0; db < DP; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) voff_[db][u] = trA_lane_off<D>(lane, 32 * db, u);
  auto koff = [&](int s) __attribute__((always_inline)) { return koff_[s % KP] + (s / KP) * (16 * KP); };
  auto voff = [&](int db, int u) __attribute__((always_inline)) { return voff_[db % DP][u] + (db / DP) * (32 * DP); };

  // Prologue: the first NBUF - 1 tiles in flight, the first one landed.
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < ntiles) issue_tile(j, j);
  wait_tiles<NBUF - 2, Tile::PER>(ntiles > NBUF - 2 ? NBUF - 2 : ntiles - 1);
  __syncthreads();

  // One tile; BUF (the LDS buffer holding it) is a compile-time constant so
  // that every LDS read below is a lane register plus an immediate offset.
  auto tile = [&](auto bufc, int i) __attribute__((always_inline)) {
    constexpr int BUFI = decltype(bufc)::value;
    // refill the buffer read in the previous iteration, NBUF - 1 tiles ahead
    const int ahead = i + NBUF - 1;
    if (ahead < ntiles) issue_tile(ahead, (BUFI + NBUF - 1) % NBUF);
    const uint16_t* Ks = smem + BUFI * C::BUF;
    const uint16_t* Vs = Ks + Tile::ELEMS;

    if (wave_active) {
      const bool second = i >= n0;
      const int k0 = (second ? seg.begin1 + (i - n0) : seg.begin0 + i) * BN;
      int lf, hf, ll, hl, lo, hi;
      if constexpr (D >= 192 || BN == 32) {
        const int kh = second ? seg.half1 : seg.half0;
        row_interval_of_block(qh, kh, bs_f, be_f, lf, hf);
        row_interval_of_block(qh, kh, bs_l, be_l, ll, hl);
        row_interval_of_block(qh, kh, bs_p, be_p, lo, hi);
      } else {
        lf = second ? lo_f1 : lo_f0;
        hf = second ? hi_f1 : hi_f0;
        ll = second ? lo_l1 : lo_l0;
        hl = second ? hi_l1 : hi_l0;
        lo = second ? lo_p1 : lo_p0;
        hi = second ? hi_p1 : hi_p0;
      }
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
        mfma_burst_begin();
#pragma unroll
        for (int s = 0; s < C::KS; ++s) acc = mfma32(lds_vec_at(Ks + 32 * kb * D + koff(s)), qf[s], acc);
        mfma_burst_end();
        if constexpr (SC) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = softcap_y(capc, softcap_r(capc, acc[r]));
        }
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
        lr_run *= alpha;
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
        const bf16x8 pb0 = pack_bf16x8(sc[kb], 0), pb1 = pack_bf16x8(sc[kb], 8);
        lr_run = sum_bf16x8(pb0, sum_bf16x8(pb1, lr_run));
        mfma_burst_begin();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint16_t* vrow = Vs + (32 * kb + 16 * ks) * D;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            o[db] = mfma32(lds_trA_at(vrow + voff(db, 0), vrow + voff(db, 1)), ks ? pb1 : pb0, o[db]);
        }
        mfma_burst_end();
      }
    }

    // tile i + 1 must have landed; later ones may stay in flight
    const int in_flight = min(ntiles - 1, i + NBUF - 1) - (i + 1);
    wait_tiles<NBUF - 2, Tile::PER>(in_flight);
    __syncthreads();
  };

  static_assert(NBUF >= 2 && NBUF <= 4, "ring of two to four tiles");
  for (int i = 0; i < ntiles; i += NBUF) {
    static_for<NBUF>([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      if (i + J < ntiles) tile(std::integral_constant<int, J>{}, i + J);
    });
  }

  // Epilogue: O = z / l~, LSE = (m + log2 l) * ln 2.  z sums the bf16
  // probabilities times V, so dividing by their own sum l~ makes O a
  // weighted average of the V rows with weights that sum to one: the
  // rounding of P then moves O by at most 2^-9 sum_j w_j |v_j - O| instead
  // of 2^-9 sum_j w_j |v_j| (which, in a row dominated by one key whose
  // probability was rounded above a stale maximum, approaches 2^-9 |O|).
  // The LSE keeps the float32 sum.
  const float l_tot = halves_sum(l_run);
  if (wave_active && p < n) {
    const float inv = 1.f / halves_sum(lr_run);
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
      a.lse[stat0 + (size_t)hh * a.stat_hs + qoff + p] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, int BN, int NW = 4, int NBUF = 2>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t s) {
  using C = FwdCfg<D, BN, NW, NBUF>;
  const int qtiles = (a.n + C::BM - 1) / C::BM;
  const long long blocks = (long long)qtiles * a.nhalves * a.B * a.H;
  if (a.softcap > 0.f)
    hipLaunchKernelGGL((fwd_kernel<D, BN, NW, NBUF, true>), dim3((unsigned)blocks), dim3(C::NT), 0, s, a, qtiles);
  else
    hipLaunchKernelGGL((fwd_kernel<D, BN, NW, NBUF, false>), dim3((unsigned)blocks), dim3(C::NT), 0, s, a, qtiles);
  return hipGetLastError();
}

#ifndef BDATTN_FWD_NW
#define BDATTN_FWD_NW 4
#endif
#ifndef BDATTN_FWD_BN
#define BDATTN_FWD_BN 64
#endif
#ifndef BDATTN_FWD_NBUF
#define BDATTN_FWD_NBUF 2
#endif

hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t s) {
  if (D == 64) return launch_fwd_t<64, BDATTN_FWD_BN, BDATTN_FWD_NW, BDATTN_FWD_NBUF>(a, s);
  if (D == 96) return launch_fwd_t<96, 64, 4, 2>(a, s);
  if (D == 192) return launch_fwd_t<192, 32, 4, 2>(a, s);
  if (D == 256) return launch_fwd_t<256, 32, 4, 2>(a, s);
  return launch_fwd_t<128, 32, 4, 2>(a, s);
}

}  // namespace bd
