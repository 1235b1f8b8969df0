// attn_bwd.hip -- backward pass, split in two kernels:
//
//   dq   : one workgroup per 128-row query tile.  Each wave first computes,
//          for its 32 rows, delta_i = dO_i . O_i and lse_i * log2(e) and
//          stores -delta and lse2 (float32) in the caller's workspace; then
//          it walks the key tiles its rows see and accumulates
//          dQ = scale * dS K;
//   dkdv : one workgroup per key tile of one key/value head (192 keys for
//          multi-head D = 128, 64 at D = 256, 128 otherwise; runs after dq,
//          reading the workspace); it walks the query tiles that
//          see its keys, for every query head that reads the key/value head
//          in turn, and accumulates dV = P^T dO and dK = scale * dS^T Q in
//          registers.  With grouped query heads the key tile is loaded once
//          for the whole group and the group's sum needs no atomics (Fast
//          Diffusion Attention, "Ampere and Ada": the GQA-grouped backward).
//
// FlashAttention: Exact Attention Without Materialization, section 4.5:
// the probabilities are recomputed on chip from Q, K and the saved
// log-sum-exp (P = exp(scale * q.k - LSE)) rather than stored.  With
// dP = dO V^T, dS = P * (dP - delta).  Fast Diffusion Attention, "Visit only
// the visible tiles": each key tile visits exactly the query tiles that see
// it (geometry.h, bwd_segments), each query tile exactly the key tiles it
// sees.  Neither kernel uses atomics, so the result is deterministic.
//
// Mapping to gfx950 (MFMA layouts in common.h, LDS tiles in tile_io.h):
//  dkdv: each pair of waves owns 32 keys, one holding K and the other V as
//    B operands in registers for the whole walk.  S = Q K^T and dP = dO V^T come out with
//    one key per lane and the query rows in registers; read with k = query
//    row they are directly the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands come from the natural Q and dO tiles
//    through transposing LDS reads.
//  dq: each wave owns 32 query rows and holds Q and dO as B operands.
//    S^T = K Q^T and dP^T = V dO^T give one query per lane, so the row
//    statistics are per-lane scalars; dQ^T += K^T dS^T reads K^T from the
//    natural K tile through transposing reads.
//  Both stream their tiles with buffer loads that write LDS directly,
//  double-buffered, one tile ahead.
#include "common.h"
#include "geometry.h"
#include "kernels.h"
#include "tile_io.h"

#include <type_traits>

namespace bd {

// Token offset of a half inside its sample (n: the sample's half length).
__device__ __forceinline__ int half_off(const AttnArgs& a, int half, int n) {
  return (a.mode == MODE_DIFFUSION && half == CLEAN) ? n : 0;
}

// Per-segment scalars.  A key-stationary wave needs, for each query half it
// walks, the rows that see this lane's key (element mask), the offsets of
// row 0 of Q / dO and of its statistics, and the rows that see its first and
// last keys (query-block classification).  A query-stationary wave needs the
// visible intervals of its first, last and own rows and the offset of row 0
// of K / V.  They are kept as separate scalars and picked with selects:
// grouped in a struct, the compiler would select between the structs'
// addresses and keep both in scratch memory.
#define COL_SEGMENTS                                                          \
  const size_t stat_base = stat0 + (size_t)hh0 * a.stat_hs;                  \
  int clo_p0, chi_p0, clo_p1, chi_p1;                                        \
  col_interval(g, seg.half0, kh, key, clo_p0, chi_p0);                        \
  col_interval(g, seg.half1, kh, key, clo_p1, chi_p1);                        \
  const size_t qb0 = (sample0 + half_off(a, seg.half0, n)) * rs + (size_t)hh0 * D; \
  const size_t qb1 = (sample0 + half_off(a, seg.half1, n)) * rs + (size_t)hh0 * D; \
  const size_t sb0 = stat_base + half_off(a, seg.half0, n);                   \
  const size_t sb1 = stat_base + half_off(a, seg.half1, n);

#define ROW_SEGMENTS                                                           \
  constexpr bool ROW_BLOCKS = D >= 192;  /* per-tile intervals from the rows' blocks */ \
  const int bs_f = ROW_BLOCKS ? g.bstart(pw0) : 0, be_f = ROW_BLOCKS ? g.bend(pw0) : 0; \
  const int bs_l = ROW_BLOCKS ? g.bstart(max(pw1 - 1, pw0)) : 0;               \
  const int be_l = ROW_BLOCKS ? g.bend(max(pw1 - 1, pw0)) : 0;                 \
  const int bs_p = ROW_BLOCKS ? g.bstart(p) : 0, be_p = ROW_BLOCKS ? g.bend(p) : 0; \
  int lo_f0, hi_f0, lo_l0, hi_l0, lo_p0, hi_p0, lo_f1, hi_f1, lo_l1, hi_l1, lo_p1, hi_p1; \
  row_interval(g, qh, seg.half0, pw0, lo_f0, hi_f0);                            \
  row_interval(g, qh, seg.half0, max(pw1 - 1, pw0), lo_l0, hi_l0);              \
  row_interval(g, qh, seg.half0, p, lo_p0, hi_p0);                              \
  row_interval(g, qh, seg.half1, pw0, lo_f1, hi_f1);                            \
  row_interval(g, qh, seg.half1, max(pw1 - 1, pw0), lo_l1, hi_l1);              \
  row_interval(g, qh, seg.half1, p, lo_p1, hi_p1);                              \
  const size_t kvb0 = (sample0 + half_off(a, seg.half0, n)) * rs_kv + (size_t)hk * D; \
  const size_t kvb1 = (sample0 + half_off(a, seg.half1, n)) * rs_kv + (size_t)hk * D;

// ---------------------------------------------------------------------------
// dK / dV of the noisy keys: the block diagonal of the noisy half.
// ---------------------------------------------------------------------------
// Fast Diffusion Attention, "Hopper": the noisy diagonal of the backward
// pass has a kernel of its own, and the main dK/dV kernel walks the clean
// key tiles only.  A noisy key is seen by the noisy queries of its own block
// and by no other query ("Block diffusion in one picture"), so its dK and dV
// are sums over that block's rows alone.  Each wave owns 32 keys and works
// alone (no barrier, no exchange with other waves): it holds K and V as B
// operands, stages the rows of its keys' blocks 32 at a time (Q and dO) in
// its own LDS region, and per 32-row chunk computes S = Q K^T, P from the
// saved LSE, dP = dO V^T, dS = P (dP - delta), dV^T += dO^T P and
// dK^T += Q^T dS (FlashAttention: Exact Attention Without Materialization,
// section 4.5), one key per lane as in the main kernel.  With grouped heads
// the wave walks every query head of the group, so dK and dV are written
// once, in bf16, without partials.
// The dedicated kernel is a build option (BDATTN_NOISY_DIAG_KERNEL, off by
// default): on MI355X the main kernel's own noisy key tiles measured faster
// at every workload tried (its paired waves skip the invisible 32 x 32
// blocks, and its light noisy workgroups fill the tail of the launch, which
// a second launch cannot).  With the option, blocks up to kDiagMaxBlock use
// it; above, a noisy key tile is seen by many rows and the main kernel
// walks it as usual.
constexpr int kDiagMaxBlock = 64;

__host__ __device__ inline bool use_noisy_diag(int mode, int b) {
#ifdef BDATTN_NOISY_DIAG_KERNEL
  return mode == MODE_DIFFUSION && b <= kDiagMaxBlock;
#else
  (void)mode;
  (void)b;
  return false;
#endif
}

// One wave, keys [k0, k0 + 32) of the noisy half of sample bi, key/value
// head hk (every query head of its group in turn): pass 0 sums
// dV^T += dO^T P, pass 1 dK^T += Q^T dS (two waves share the work of one
// group of keys, so that only one accumulator set is live in each).  Tq
// and Tg: the wave's LDS regions for 32 rows of Q and of dO.
template <int D, bool GROUPED, bool SC>
__device__ __forceinline__ void noisy_diag_wave(const AttnArgs& a, int bi, int hk, int k0, int pass,
                                                uint16_t* Tq, uint16_t* Tg, int lane) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using Tile = DirectTile<32, D, 64>;  // one wave's 32-row chunk
  const int l32 = lane & 31;
  const int h2 = lane >> 5;
  size_t sample0, stat0;
  int n;
  if (!sample_of(a, bi, sample0, n, stat0) || k0 >= n) return;
  const Geom g{n, a.b};
  const int key = k0 + l32;
  // the rows that see some key of the wave, and those that see this lane's
  const int r_lo = g.bstart(k0);
  const int r_hi = g.bend(min(k0 + 31, n - 1));
  const int clo = key < n ? g.bstart(key) : 0;
  const int chi = key < n ? g.bend(key) : 0;

  const size_t rs = (size_t)a.H * D;
  const size_t rs_kv = (size_t)a.Hkv * D;
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const uint32_t half_bytes = (uint32_t)n * row_bytes;
  const uint32_t kv_row_bytes = (uint32_t)rs_kv * 2u;

  const size_t kb = sample0 * rs_kv + (size_t)hk * D;
  const rsrc_t rk = make_rsrc(a.k + kb, (uint32_t)n * kv_row_bytes);
  const rsrc_t rv = make_rsrc(a.v + kb, (uint32_t)n * kv_row_bytes);
  const uint32_t lq = __builtin_amdgcn_readfirstlane(lds_byte_addr(Tq));
  const uint32_t lg = __builtin_amdgcn_readfirstlane(lds_byte_addr(Tg));
  const Softcap capc = SC ? softcap_consts(a.scale, a.softcap) : Softcap{0.f, 0.f};
  const int G = GROUPED ? a.G : 1;
  {
    bf16x8 xk[KS], xv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = (uint32_t)key * kv_row_bytes + (uint32_t)(16 * s + 8 * h2) * 2u;
      xk[s] = as_bf16x8(buf_ld16(rk, off, 0));
      if (pass == 1) xv[s] = as_bf16x8(buf_ld16(rv, off, 0));
    }
    floatx16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = zero16();
    for (int gi = 0; gi < G; ++gi) {
      const int hh = hk * G + gi;
      const size_t qb = sample0 * rs + (size_t)hh * D;
      const rsrc_t rq = make_rsrc(a.q + qb, half_bytes);
      const rsrc_t rg = make_rsrc(a.dout + qb, half_bytes);
      const size_t sb = stat0 + (size_t)hh * a.stat_hs;
      const rsrc_t rl = make_rsrc(a.lse2 + sb, (uint32_t)n * 4u);
      const rsrc_t rd = make_rsrc(a.ndelta + sb, (uint32_t)n * 4u);
      for (int r0 = r_lo; r0 < r_hi; r0 += 32) {
        // the previous chunk's LDS reads are over (their values fed the
        // products below); refill the wave's regions
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        Tile::load(rq, row_bytes, r0, lq, lane);
        Tile::load(rg, row_bytes, r0, lg, lane);
        wait_vmem();
        // S = Q K^T (and dP = dO V^T in pass 1); register r holds row
        // r0 + 8 (r / 4) + 4 h2 + r % 4; rows past the half read lse2 =
        // -delta = 0 (and Q = dO = 0)
        floatx16 sc = zero16(), dp;
        if (pass == 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dp[r] = buf_ldf(rd, (uint32_t)(r0 + 8 * (r >> 2) + 4 * h2 + (r & 3)) * 4u);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sc = mfma32(lds_vec_at(Tq + row8_lane_off<D>(lane, 2 * s)), xk[s], sc);
          if (pass == 1) dp = mfma32(lds_vec_at(Tg + row8_lane_off<D>(lane, 2 * s)), xv[s], dp);
        }
        // P (zero where the row is outside this lane's key's block), or dS
        floatx16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const float l2 = buf_ldf(rl, (uint32_t)row * 4u);
          float p;
          if constexpr (SC) {
            const float rr = softcap_r(capc, sc[r]);
            p = fast_exp2(softcap_y(capc, rr) - l2);
            if (pass == 1) p *= 4.f * rr * (1.f - rr) * dp[r];
          } else {
            p = fast_exp2(__builtin_fmaf(sc[r], a.scale_log2, -l2));
            if (pass == 1) p *= dp[r];
          }
          x[r] = (row >= clo && row < chi) ? p : 0.f;
        }
        const bf16x8 xb[2] = {pack_bf16x8(x, 0), pack_bf16x8(x, 8)};
        // pass 0: dV^T += dO^T P; pass 1: dK^T += Q^T dS
        const uint16_t* T = pass == 0 ? Tg : Tq;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint16_t* tr = T + 16 * ks * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32(lds_trA_at(tr + trA_lane_off<D>(lane, 32 * db, 0), tr + trA_lane_off<D>(lane, 32 * db, 1)),
                             xb[ks], acc[db]);
        }
      }
    }
    // lane = key, register r of block db = dimension 32db + 8(r/4) + 4h2 + r%4
    if (key < n) {
      const size_t off = (sample0 + key) * rs_kv + (size_t)hk * D;
      uint16_t* dst = (pass == 0 ? a.dv : a.dk) + off;
      const float f = pass == 0 ? 1.f : a.scale;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * h2;
          u32x2 pk = {pack2_bf16(acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f),
                      pack2_bf16(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
          *reinterpret_cast<u32x2*>(dst + d) = pk;
        }
    }
  }
}


// 4 waves, 64 keys: waves 0 and 1 sum dV for keys 64 kt + 32 w, waves 2
// and 3 dK for the same keys.  Each wave has 32 rows of Q and of dO in LDS.
template <int D>
struct DiagCfg {
  static constexpr int NT = 256;
  static constexpr int BKV = 64;
  static constexpr int CH = 32 * D;  // elements of one 32-row chunk
};

template <int D, bool GROUPED, bool SC>
__global__ __launch_bounds__(DiagCfg<D>::NT, 1) void bwd_noisy_diag_kernel(AttnArgs a, int dtiles) {
  using C = DiagCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * 2 * C::CH];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int BH = a.B * a.Hkv;
  const int kt = blockIdx.x / BH;
  const int bi = (blockIdx.x % BH) / a.Hkv;
  const int hk = (blockIdx.x % BH) % a.Hkv;
  uint16_t* T = smem + 2 * wv * C::CH;
  noisy_diag_wave<D, GROUPED, SC>(a, bi, hk, kt * C::BKV + 32 * (wv & 1), wv >> 1, T, T + C::CH,
                                  threadIdx.x & 63);
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary, one pair of waves per 32 keys; four pairs (128
// keys, 8 waves) per workgroup unless stated below.
// The pair's two waves share 32 keys: the P-wave holds K and computes
// S = Q K^T, P and dV^T += dO^T P; the dS-wave holds V and computes
// dP = dO V^T, dS = P (dP - delta) and dK^T += Q^T dS.  The dS-wave needs the
// P-wave's probabilities, so it runs one query tile behind: in step j the
// P-wave works on tile j and publishes its P (bf16) in LDS, while the
// dS-wave works on tile j - 1 with the P published in step j - 1.  One
// workgroup barrier per step orders everything: the Q / dO ring holds the
// P-waves' tile, the dS-waves' tile and the tile in flight, and the P
// exchange is double-buffered.
// ---------------------------------------------------------------------------
// D = 192 and 256 stream 32-row query tiles, so that the three-deep Q / dO
// ring fits LDS; D = 256 also runs two pairs only (one wave per SIMD, each
// with the whole register file), while D = 192 still fits two waves per SIMD.
// D = 64 streams 32-row tiles too: its LDS (42 KiB) and registers (at most
// 128) then fit two workgroups per CU, four waves per SIMD.  So does D = 96
// (54 KiB), except with softcapping, whose extra per-score work does not fit
// 128 registers: that instance keeps 64-row tiles at one workgroup per CU.
// Multi-head D = 128 streams 32-row tiles with six pairs (12 waves, 192
// keys): with 32-row steps a wave needs at most 168 registers, so three waves
// share a SIMD, and every Q / dO tile serves 192 keys instead of 128 (dK/dV
// 3% faster than four pairs with 64-row steps on 2 x 8192 x 32 heads,
// 8 x 2048 x 16 and 4 x 4096 x 16).  Grouped heads keep four pairs: a grouped
// workgroup walks G query heads, so its grid is G times coarser, and 192-key
// workgroups left a ragged last round (2 x 8192 tokens, 32 heads over 8
// key/value heads: 13% slower).  At D = 64 one workgroup of eight pairs was
// 8-18% slower than two of four.
template <int D, bool SC = false, bool GROUPED = false>
struct DkdvCfg {
  static constexpr bool WIDE = D >= 192;
  static constexpr bool SHORT = D == 64 || (D == 96 && !SC);  // 32-row tiles, two workgroups per CU
  static constexpr bool SIX = D == 128 && !GROUPED;  // 32-row tiles, six pairs, three waves per SIMD
  static constexpr int WGS = SHORT ? 2 : 1;  // workgroups per CU
  static constexpr int NPAIR = D == 256 ? 2 : SIX ? 6 : 4;
  static constexpr int NT = 128 * NPAIR;  // 8 waves (12 at D = 128, 4 at D = 256)
  static constexpr int BKV = 32 * NPAIR;  // keys per workgroup
  static constexpr int BQ = (WIDE || SHORT || SIX) ? 32 : 64;  // query rows per streamed tile
  static constexpr int QB = BQ / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NBUF = 3;          // Q / dO ring depth
  // The P-waves (threads [0, NT / 2)) load the tiles: they finish their
  // share of a step earlier, so they also absorb the wait for the next
  // tile, and the barrier that ends the step publishes it to the dS-waves.
  using Tile = DirectTile<BQ, D, NT / 2>;
  static constexpr int BUF = 2 * Tile::ELEMS;   // Q then dO
  // lse2 then -delta, each loaded by one wave-wide instruction (64 floats)
  static constexpr int STATW = 64;
  static constexpr int FBUF = 2 * STATW;
  static constexpr int PXS = NPAIR * QB * 2 * 64;  // 16-byte slots of one P exchange buffer
};

// GROUPED: G > 1 query heads per key/value head (the walk spans several
// query heads, and with S > 1 the workgroup writes float32 partials); the
// plain multi-head instance compiles none of that.  SC: softcapping on (the
// P-wave recomputes P from the capped scores and publishes
// P (1 - tanh^2), so that the dS-wave's dS carries the cap's derivative).
template <int D, bool GROUPED, bool SC>
__global__ __launch_bounds__((DkdvCfg<D, SC, GROUPED>::NT), (DkdvCfg<D, SC, GROUPED>::WGS)) void bwd_dkdv_kernel(
    AttnArgs a, int ktiles) {
  using C = DkdvCfg<D, SC, GROUPED>;
  static_assert(C::NT == DkdvCfg<D, false, GROUPED>::NT && C::BKV == DkdvCfg<D, false, GROUPED>::BKV,
                "one grid with and without the cap");
  using Tile = typename C::Tile;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::NBUF * C::BUF];
  __shared__ __attribute__((aligned(16))) float fsm[C::NBUF * C::FBUF];
  __shared__ __attribute__((aligned(16))) u32x4 pex[2 * C::PXS];
  const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_byte_addr(smem));
  const uint32_t fbase = __builtin_amdgcn_readfirstlane(lds_byte_addr(fsm));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wv % C::NPAIR;
  const bool pwave = wv < C::NPAIR;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // One workgroup per (key tile, sample, key/value head, split); it walks
  // the query tiles of the G / S query heads of its split of the group (the
  // grouped backward: the key tile is loaded once for all of them).
  const int S = GROUPED ? a.S : 1;
  const int BH = a.B * a.Hkv * S;
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
  const int split = GROUPED ? bh % S : 0;
  const int bi = bh / S / a.Hkv;
  const int hk = bh / S % a.Hkv;
  const int gs = GROUPED ? a.G / S : 1;         // query heads walked by this workgroup
  const int hh0 = GROUPED ? hk * a.G + split * gs : hk;  // the first of them
  size_t sample0, stat0;
  int n;
  // packed samples shorter than the longest leave their last tiles empty
  if (!sample_of(a, bi, sample0, n, stat0) || kt * C::BKV >= n) return;
  const Geom g{n, a.b};
  // Q / dO rows hold H heads, K / V / dK / dV rows Hkv heads.
  const size_t rs = (size_t)a.H * D;
  const size_t rs_kv = (size_t)a.Hkv * D;
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const uint32_t half_bytes = (uint32_t)n * row_bytes;
  const uint32_t kv_row_bytes = (uint32_t)rs_kv * 2u;
  const size_t koff = sample0 + half_off(a, kh, n);

  const int kw0 = kt * C::BKV + 32 * pair;  // the pair's first key
  const int kw1 = min(kw0 + 32, n);
  const bool pair_active = kw0 < n;
  const int key = kw0 + l32;

  // The P-wave holds K, the dS-wave V, as B operands.
  bf16x8 xf[C::KS];
  {
    const rsrc_t rx = make_rsrc((pwave ? a.k : a.v) + koff * rs_kv + (size_t)hk * D,
                                (uint32_t)n * kv_row_bytes);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      xf[s] = as_bf16x8(buf_ld16(rx, (uint32_t)key * kv_row_bytes + (uint32_t)(16 * s + 8 * h2) * 2u, 0));
#pragma unroll
    for (int s = 0; s < C::KS; ++s) settle(xf[s]);
  }

  const Segments seg = bwd_segments(g, a.mode, kh, kt, C::BQ, C::BKV);
  const int n0 = seg.count > 0 ? seg.end0 - seg.begin0 : 0;
  const int ntiles = seg.tiles();
  // Step t of the walk is tile t mod ntiles of query head hh0 + t / ntiles.
  const int nsteps = gs * ntiles;
  auto head_of_step = [&](int t) -> int { return (!GROUPED || gs == 1) ? 0 : t / ntiles; };
  COL_SEGMENTS
  // the blocks of the pair's first and last keys
  const int kblk_f0 = g.bstart(kw0), kblk_f1 = g.bend(kw0);
  const int kblk_l0 = g.bstart(max(kw1 - 1, kw0)), kblk_l1 = g.bend(max(kw1 - 1, kw0));
  int clo_f0, chi_f0, clo_l0, chi_l0, clo_f1, chi_f1, clo_l1, chi_l1;
  col_interval_of_block(n, seg.half0, kh, kblk_f0, kblk_f1, clo_f0, chi_f0);
  col_interval_of_block(n, seg.half0, kh, kblk_l0, kblk_l1, clo_l0, chi_l0);
  col_interval_of_block(n, seg.half1, kh, kblk_f0, kblk_f1, clo_f1, chi_f1);
  col_interval_of_block(n, seg.half1, kh, kblk_l0, kblk_l1, clo_l1, chi_l1);
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int gi = head_of_step(t);
    const int i = t - gi * ntiles;
    const bool second = i >= n0;
    const int qt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
    const size_t qb = (second ? qb1 : qb0) + (size_t)gi * D;
    const size_t sb = (second ? sb1 : sb0) + (size_t)gi * a.stat_hs;
    const uint32_t dst = sbase + (uint32_t)(buf * C::BUF) * 2u;
    Tile::load(make_rsrc(a.q + qb, half_bytes), row_bytes, qt * C::BQ, dst, tid);
    Tile::load(make_rsrc(a.dout + qb, half_bytes), row_bytes, qt * C::BQ, dst + Tile::ELEMS * 2u, tid);
    // rows past the half read lse2 = -delta = 0; their Q and dO rows are
    // zero too, so they add nothing to dV or dK
    const uint32_t sbytes = (uint32_t)n * 4u;
    const uint32_t fdst = fbase + (uint32_t)(buf * C::FBUF) * 4u;
    if (wv == 0)
      lds_direct4(make_rsrc(a.lse2 + sb, sbytes), fdst, (uint32_t)lane * 4u, (uint32_t)qt * C::BQ * 4u);
    if (wv == 1)
      lds_direct4(make_rsrc(a.ndelta + sb, sbytes), fdst + C::STATW * 4u, (uint32_t)lane * 4u,
                  (uint32_t)qt * C::BQ * 4u);
  };

  floatx16 acc[C::DB];  // dV (P-wave) or dK (dS-wave)
#pragma unroll
  for (int i = 0; i < C::DB; ++i) acc[i] = zero16();

  if (pwave && nsteps > 0) issue_tile(0, 0);
  wait_vmem();
  __syncthreads();

  // The two roles run separate copies of the walk, so that each is
  // register-allocated for its own state only.  Both pass one workgroup
  // barrier per step, nsteps + 1 steps.  In step j the P-wave computes S, P
  // and dV for tile j (products, elementwise, products); the dS-wave first
  // finishes tile j - 1 (dS from the dP it computed in the previous step,
  // then dK) and then computes dP for tile j.  Waves go to the SIMDs in turn,
  // so with four pairs the two waves of a pair (w and w + 4) share a SIMD,
  // and this order puts one wave's elementwise work beside the other's
  // products; with six, a SIMD holds three waves of different pairs.
  auto walk = [&](auto rolec) __attribute__((always_inline)) {
    constexpr bool PW = decltype(rolec)::value;
    // Per-lane LDS offsets (elements from the start of a buffer), fixed for
    // the walk: the first product reads the wave's A operand tile (Q for the
    // P-wave, dO for the dS-wave) row-wise, the second reads the other tile
    // transposed.
    constexpr int xsel = PW ? 0 : Tile::ELEMS;
    constexpr int ysel = PW ? Tile::ELEMS : 0;
    int xoff[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) xoff[s] = xsel + row8_lane_off<D>(lane, 2 * s);
    int yoff[C::DB][2];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) yoff[db][u] = ysel + trA_lane_off<D>(lane, 32 * db, u);

    // Which 32-row blocks of tile i see some key of the pair (act) or every
    // key of it (full); qt, and the rows [clo, chi) that see this lane's key.
    auto blocks = [&](int t, bool (&act)[C::QB], bool (&full)[C::QB], int& qt, int& clo, int& chi)
        __attribute__((always_inline)) {
      const int i = t - head_of_step(t) * ntiles;
      const bool second = i >= n0;
      qt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
      // The pair's intervals for the tile's half.  With 32-row tiles they
      // are derived here: selected from the two halves' copies, they ended
      // up read through a table of addresses in scratch memory.  (The copies
      // measured slightly faster at the other widths.)
      int cf, hf, cl, hl;
      if constexpr (C::BQ == 32) {
        const int qh = second ? seg.half1 : seg.half0;
        col_interval_of_block(n, qh, kh, kblk_f0, kblk_f1, cf, hf);
        col_interval_of_block(n, qh, kh, kblk_l0, kblk_l1, cl, hl);
      } else {
        cf = second ? clo_f1 : clo_f0;
        hf = second ? chi_f1 : chi_f0;
        cl = second ? clo_l1 : clo_l0;
        hl = second ? chi_l1 : chi_l0;
      }
      clo = second ? clo_p1 : clo_p0;
      chi = second ? chi_p1 : chi_p0;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const int r0 = qt * C::BQ + 32 * qb;
        const int r1 = min(r0 + 32, n);
        act[qb] = pair_active && r0 < n && r1 > cf && r0 < hl;
        full[qb] = r0 >= cl && r1 <= hf;
      }
    };

    // First product of the active blocks of the tile at Tb: S^T (P-wave)
    // or dP^T (dS-wave), one key per lane.  With both blocks the two chains
    // are interleaved and the operand reads run PF steps ahead of the
    // products, an order pinned with scheduling barriers (left alone, the
    // scheduler keeps two reads in flight and every product waits for its
    // read).
    //
    // The accumulators start at init(qb): zero for S; for dP the rows'
    // -delta, so that the chain yields dP - delta.
    auto product1 = [&](const uint16_t* Tb, const bool (&act)[C::QB], floatx16 (&t)[C::QB], auto init)
        __attribute__((always_inline)) {
      mfma_burst_begin();
      if constexpr (C::QB == 2) {
        if (act[0] && act[1]) {
        constexpr int PF = 2;
        t[0] = init(0);
        t[1] = init(1);
        bf16x8 a0[C::KS], a1[C::KS];
#pragma unroll
        for (int s = 0; s < PF; ++s) {
          a0[s] = lds_vec_at(Tb + xoff[s]);
          a1[s] = lds_vec_at(Tb + 32 * D + xoff[s]);
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          if (s + PF < C::KS) {
            a0[s + PF] = lds_vec_at(Tb + xoff[s + PF]);
            a1[s + PF] = lds_vec_at(Tb + 32 * D + xoff[s + PF]);
          }
          t[0] = mfma32(a0[s], xf[s], t[0]);
          t[1] = mfma32(a1[s], xf[s], t[1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_burst_end();
        return;
        }
      }
      // One block per step: at D = 256 (one wave per SIMD, nothing else to
      // cover a read's latency) the reads run two products ahead too (dK/dV
      // 4% faster at 4 x 4096 tokens, 8 heads); at D = 64, 128 and 192 the
      // same order measured within noise, so it is left to the scheduler.
      if constexpr (C::QB == 1 && D == 256) {
        if (act[0]) {
          constexpr int PF = 2;
          t[0] = init(0);
          bf16x8 a0[C::KS];
#pragma unroll
          for (int s = 0; s < PF; ++s) a0[s] = lds_vec_at(Tb + xoff[s]);
#pragma unroll
          for (int s = 0; s < C::KS; ++s) {
            if (s + PF < C::KS) a0[s + PF] = lds_vec_at(Tb + xoff[s + PF]);
            t[0] = mfma32(a0[s], xf[s], t[0]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        mfma_burst_end();
        return;
      }
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        if (!act[qb]) continue;
        t[qb] = init(qb);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) t[qb] = mfma32(lds_vec_at(Tb + 32 * qb * D + xoff[s]), xf[s], t[qb]);
      }
      mfma_burst_end();
    };
    // Second product: dV^T += dO^T P (P-wave) or dK^T += Q^T dS (dS-wave)
    // for block qb of the tile at Tb, B operand halves bop.
    auto product2 = [&](const uint16_t* Tb, auto qbc, const bf16x8 (&bop)[2]) __attribute__((always_inline)) {
      constexpr int qb = decltype(qbc)::value;
      mfma_burst_begin();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint16_t* yr = Tb + (32 * qb + 16 * ks) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          acc[db] = mfma32(lds_trA_at(yr + yoff[db][0], yr + yoff[db][1]), bop[ks], acc[db]);
      }
      mfma_burst_end();
    };

    // dS-wave: dP of the previous tile and which of its blocks are active
    floatx16 dpr[C::QB];
    bool pact[C::QB] = {};
    // Step j; tile j sits in ring slot SLOT = j mod NBUF, a compile-time
    // constant (the loop below is unrolled by the ring depth) so that every
    // LDS read is a lane register plus an immediate offset.
    auto step_j = [&](auto slotc, int j) __attribute__((always_inline)) {
      constexpr int slot = decltype(slotc)::value;
      constexpr int slot_next = (slot + 1) % C::NBUF;
      constexpr int slot_prev = (slot + C::NBUF - 1) % C::NBUF;
      if (PW && j + 1 < nsteps) issue_tile(j + 1, slot_next);
      if constexpr (PW) {
        if (j < nsteps) {
          const uint16_t* Tb = smem + slot * C::BUF;
          const float* Ls = fsm + slot * C::FBUF;
          u32x4* px = pex + (j & 1) * C::PXS + pair * (C::QB * 2 * 64) + lane;
#ifdef BDATTN_LDS_POISON
          // the dS-wave finished reading this exchange buffer (step j - 2's
          // P) before the barrier that started this step
#pragma unroll
          for (int u = 0; u < C::QB * 2; ++u) px[u * 64] = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
          bool act[C::QB], full[C::QB];
          int qt, clo, chi;
          blocks(j, act, full, qt, clo, chi);
          floatx16 t[C::QB];
          product1(Tb, act, t, [](int) { return zero16(); });
          // P = exp2(S * scale * log2 e - LSE * log2 e), published for the
          // dS-wave of the pair (read in the next step)
          auto step = [&](auto qbc) __attribute__((always_inline)) {
            constexpr int qb = decltype(qbc)::value;
            if (!act[qb]) return;
            floatx16& x = t[qb];
            floatx16 dc;  // softcapping: 1 - tanh^2 of each score
            if constexpr (SC) {
              const Softcap capc = softcap_consts(a.scale, a.softcap);
#pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const float4 l4 = *reinterpret_cast<const float4*>(Ls + 32 * qb + 8 * gq + 4 * h2);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  const float rr = softcap_r(capc, x[4 * gq + u]);
                  x[4 * gq + u] = fast_exp2(softcap_y(capc, rr) - lv[u]);
                  dc[4 * gq + u] = 4.f * rr * (1.f - rr);
                }
              }
            } else {
#pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const float4 l4 = *reinterpret_cast<const float4*>(Ls + 32 * qb + 8 * gq + 4 * h2);
                x[4 * gq + 0] = fast_exp2(__builtin_fmaf(x[4 * gq + 0], a.scale_log2, -l4.x));
                x[4 * gq + 1] = fast_exp2(__builtin_fmaf(x[4 * gq + 1], a.scale_log2, -l4.y));
                x[4 * gq + 2] = fast_exp2(__builtin_fmaf(x[4 * gq + 2], a.scale_log2, -l4.z));
                x[4 * gq + 3] = fast_exp2(__builtin_fmaf(x[4 * gq + 3], a.scale_log2, -l4.w));
              }
            }
            if (!full[qb]) {
              // zero the rows that do not see this lane's key: register r
              // holds row r0 + 8 (r / 4) + r % 4, r0 = first row + 4 h2
              const int r0 = qt * C::BQ + 32 * qb + 4 * h2;
              const int lo = clo - r0, hi = chi - r0;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int off = 8 * (r >> 2) + (r & 3);
                x[r] = (off >= lo && off < hi) ? x[r] : 0.f;
              }
            }
            const bf16x8 bop[2] = {pack_bf16x8(x, 0), pack_bf16x8(x, 8)};
            if constexpr (SC) {
              floatx16 xd;
#pragma unroll
              for (int r = 0; r < 16; ++r) xd[r] = x[r] * dc[r];
              px[(qb * 2 + 0) * 64] = __builtin_bit_cast(u32x4, pack_bf16x8(xd, 0));
              px[(qb * 2 + 1) * 64] = __builtin_bit_cast(u32x4, pack_bf16x8(xd, 8));
            } else {
              px[(qb * 2 + 0) * 64] = __builtin_bit_cast(u32x4, bop[0]);
              px[(qb * 2 + 1) * 64] = __builtin_bit_cast(u32x4, bop[1]);
            }
            product2(Tb, qbc, bop);
          };
          static_for<C::QB>(step);
        }
      } else {
        if (j >= 1) {
          // dS = P (dP - delta) and dK for tile j - 1, P as published by the
          // P-wave (bf16); dpr already holds dP - delta
          const uint16_t* Tb = smem + slot_prev * C::BUF;
          const u32x4* px = pex + ((j - 1) & 1) * C::PXS + pair * (C::QB * 2 * 64) + lane;
          auto step = [&](auto qbc) __attribute__((always_inline)) {
            constexpr int qb = decltype(qbc)::value;
            if (!pact[qb]) return;
            floatx16& x = dpr[qb];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const u32x4 pw = px[(qb * 2 + u) * 64];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                x[8 * u + 2 * w] *= __builtin_bit_cast(float, pw[w] << 16);
                x[8 * u + 2 * w + 1] *= __builtin_bit_cast(float, pw[w] & 0xffff0000u);
              }
            }
            const bf16x8 bop[2] = {pack_bf16x8(x, 0), pack_bf16x8(x, 8)};
            product2(Tb, qbc, bop);
          };
          static_for<C::QB>(step);
        }
        if (j < nsteps) {
          bool full[C::QB];
          int qt, clo, chi;
          blocks(j, pact, full, qt, clo, chi);
          // register r of block qb holds row 32 qb + 8 (r / 4) + 4 h2 + r % 4
          const float* Nd = fsm + slot * C::FBUF + C::STATW;
          product1(smem + slot * C::BUF, pact, dpr, [&](int qb) {
            floatx16 z;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const float4 d4 = *reinterpret_cast<const float4*>(Nd + 32 * qb + 8 * gq + 4 * h2);
              z[4 * gq + 0] = d4.x;
              z[4 * gq + 1] = d4.y;
              z[4 * gq + 2] = d4.z;
              z[4 * gq + 3] = d4.w;
            }
            return z;
          });
        } else {
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) pact[qb] = false;
        }
      }
      wait_vmem();
      __syncthreads();
    };
    static_assert(C::NBUF == 3, "the step loop is unrolled by the ring depth");
    for (int j0 = 0; j0 <= nsteps; j0 += C::NBUF) {
      step_j(std::integral_constant<int, 0>{}, j0);
      if (j0 + 1 <= nsteps) step_j(std::integral_constant<int, 1>{}, j0 + 1);
      if (j0 + 2 <= nsteps) step_j(std::integral_constant<int, 2>{}, j0 + 2);
    }
  };
  if (pwave)
    walk(std::true_type{});
  else
    walk(std::false_type{});

  // lane = key, register r of block db = dimension 32db + 8(r/4) + 4h2 + r%4
  if (pair_active && key < n) {
    const size_t off = (koff + key) * rs_kv + (size_t)hk * D;
    const float f = pwave ? 1.f : a.scale;
    if (S == 1) {
      uint16_t* dst = (pwave ? a.dv : a.dk) + off;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * h2;
          u32x2 pk = {pack2_bf16(acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f),
                      pack2_bf16(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
          *reinterpret_cast<u32x2*>(dst + d) = pk;
        }
    } else {
      // float32 partial of this split: [S][B][T][Hkv][D], dK then dV
      const size_t E = (size_t)a.tokens * a.Hkv * D;
      float* dst = a.part + (pwave ? (size_t)S * E : 0) + (size_t)split * E + off;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * h2;
          float4 x = {acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f, acc[db][4 * gq + 2] * f,
                      acc[db][4 * gq + 3] * f};
          *reinterpret_cast<float4*>(dst + d) = x;
        }
    }
  }
}

// dK and dV of split groups: the sum of the S float32 partials, in split
// order, rounded to bf16.  Each thread produces 8 consecutive elements of
// the [B][T][Hkv][D] outputs; elements [0, E) are dK, [E, 2E) dV.
// With packed samples (cu non-null) only the tokens [cu[0], cu[B]) belong
// to samples: the other rows of dK and dV are left as they are.  With
// skip_noisy the rows of noisy halves are left alone too: the noisy-diagonal
// kernel writes them (T: tokens per sample when batched; packed samples
// find their sample by bisection of cu).
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part,
                                                         uint16_t* __restrict__ dk,
                                                         uint16_t* __restrict__ dv, long long E,
                                                         int S, const int* cu, int B, int row_elems,
                                                         int skip_noisy, int T) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= 2 * E) return;
  const bool second = i >= E;
  const long long e = second ? i - E : i;
  const long long t = e / row_elems;
  if (cu != nullptr) {
    if (t < cu[0] || t >= cu[B]) return;
    if (skip_noisy) {
      int lo = 0, hi = B;  // the sample s with cu[s] <= t < cu[s + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid;
      }
      if (t - cu[lo] < (cu[lo + 1] - cu[lo]) / 2) return;
    }
  } else if (skip_noisy && t % T < T / 2) {
    return;
  }
  const float* src = part + (second ? (long long)S * E : 0) + e;
  float4 lo = *reinterpret_cast<const float4*>(src);
  float4 hi = *reinterpret_cast<const float4*>(src + 4);
  for (int s = 1; s < S; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(src + (long long)s * E);
    const float4 y = *reinterpret_cast<const float4*>(src + (long long)s * E + 4);
    lo.x += x.x; lo.y += x.y; lo.z += x.z; lo.w += x.w;
    hi.x += y.x; hi.y += y.y; hi.z += y.z; hi.w += y.w;
  }
  const u32x4 pk = {pack2_bf16(lo.x, lo.y), pack2_bf16(lo.z, lo.w), pack2_bf16(hi.x, hi.y),
                    pack2_bf16(hi.z, hi.w)};
  *reinterpret_cast<u32x4*>((second ? dv : dk) + e) = pk;
}

// ---------------------------------------------------------------------------
// dQ: query-stationary.
// ---------------------------------------------------------------------------
// 4 waves at every width (at D = 192, 8 waves sharing the K / V tiles would
// need more than the 256 registers of two waves per SIMD).
template <int D>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int KB = BN / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  using Tile = DirectTile<BN, D, NT>;
  static constexpr int BUF = 2 * Tile::ELEMS;  // K then V
};

// SC: softcapping on (P from the capped scores, dS times 1 - tanh^2).
template <int D, bool SC>
__global__ __launch_bounds__(DqCfg<D>::NT, (D < 192 ? 2 : 1)) void bwd_dq_kernel(AttnArgs a, int qtiles) {
  using C = DqCfg<D>;
  using Tile = typename C::Tile;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * C::BUF];
  const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_byte_addr(smem));

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
  int bi, hh, hk;
  query_head(a, rr % BH, bi, hh, hk);
  const int qh = (a.mode == MODE_CAUSAL) ? CLEAN : half_idx;
  size_t sample0, stat0;
  int n;
  // packed samples shorter than the longest leave their last tiles empty
  if (!sample_of(a, bi, sample0, n, stat0) || qt * C::BM >= n) return;
  const Geom g{n, a.b};
  // Q / dO / O / dQ rows hold H heads, K / V rows Hkv heads.
  const size_t rs = (size_t)a.H * D;
  const size_t rs_kv = (size_t)a.Hkv * D;
  const int qoff = half_off(a, qh, n);
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const uint32_t half_bytes = (uint32_t)n * row_bytes;
  const uint32_t kv_row_bytes = (uint32_t)rs_kv * 2u;
  const uint32_t kv_half_bytes = (uint32_t)n * kv_row_bytes;

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, n);
  const bool wave_active = pw0 < n;
  const int p = pw0 + l32;

  // Q and dO as B operands: lane (row p, half h2) holds 16-byte chunks
  // 2s + h2 of its row.  Rows past the half read as zero, and so do their
  // statistics, which makes their dS zero.
  //
  // The row statistics: delta_p = dO_p . O_p from the same chunks of O
  // (FlashAttention section 4.5: rowsum(P o dP) equals dO . O), summed over
  // the lane pair (p, 0) and (p, 1); lse2_p = lse_p * log2(e).  Both go to
  // the workspace for the dK/dV kernel (-delta, so that it can start its dP
  // accumulators there).
  bf16x8 qf[C::KS], gf[C::KS];
  float lse2, ndlt;
  {
    const size_t qb = (sample0 + qoff) * rs + (size_t)hh * D;
    const rsrc_t rq = make_rsrc(a.q + qb, half_bytes);
    const rsrc_t rg = make_rsrc(a.dout + qb, half_bytes);
    const rsrc_t ro = make_rsrc(a.o + qb, half_bytes);
    u32x4 ov[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const uint32_t off = (uint32_t)p * row_bytes + (uint32_t)(16 * s + 8 * h2) * 2u;
      qf[s] = as_bf16x8(buf_ld16(rq, off, 0));
      gf[s] = as_bf16x8(buf_ld16(rg, off, 0));
      ov[s] = buf_ld16(ro, off, 0);
    }
    const size_t sb = stat0 + (size_t)hh * a.stat_hs + qoff;
    const float lse = buf_ldf(make_rsrc(a.lse_in + sb, (uint32_t)n * 4u), (uint32_t)p * 4u);
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 g = __builtin_bit_cast(u32x4, gf[s]);
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        dpart += __builtin_bit_cast(float, ov[s][w2] << 16) * __builtin_bit_cast(float, g[w2] << 16);
        dpart += __builtin_bit_cast(float, ov[s][w2] & 0xffff0000u) * __builtin_bit_cast(float, g[w2] & 0xffff0000u);
      }
    }
    ndlt = -halves_sum(dpart);
    lse2 = lse * kLog2e;
    if (wave_active && p < n && h2 == 0) {
      a.ndelta[sb + p] = ndlt;
      a.lse2[sb + p] = lse2;
    }
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      settle(qf[s]);
      settle(gf[s]);
    }
    settle(lse2);
    settle(ndlt);
  }

  const Segments seg = fwd_segments(g, a.mode, qh, qt, C::BM, BN);
  const int n0 = seg.count > 0 ? seg.end0 - seg.begin0 : 0;
  const int ntiles = seg.tiles();

  ROW_SEGMENTS
  auto issue_tile = [&](int i, int buf) __attribute__((always_inline)) {
    const bool second = i >= n0;
    const int kt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
    const size_t kvb = second ? kvb1 : kvb0;
    const uint32_t dst = sbase + (uint32_t)(buf * C::BUF) * 2u;
    Tile::load(make_rsrc(a.k + kvb, kv_half_bytes), kv_row_bytes, kt * BN, dst, tid);
    Tile::load(make_rsrc(a.v + kvb, kv_half_bytes), kv_row_bytes, kt * BN, dst + Tile::ELEMS * 2u, tid);
  };

  floatx16 dq[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) dq[i] = zero16();

  // Per-lane LDS offsets (elements from the start of a buffer): natural rows
  // of K and V (S^T = K Q^T, dP^T = V dO^T) and transposed K (dQ^T).
  // One entry per chunk position within the swizzle's span; the
  // span-multiples are compile-time offsets.
  constexpr int KP = swz_span<D>() / 2 < C::KS ? swz_span<D>() / 2 : C::KS;
  constexpr int DP = swz_span<D>() / 4 < C::DB ? swz_span<D>() / 4 : C::DB;
  int roff_[KP];
#pragma unroll
  for (int s = 0; s < KP; ++s) roff_[s] = row8_lane_off<D>(lane, 2 * s);
  int toff_[DP][2];
#pragma unroll
  for (int db = 0; db < DP; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) toff_[db][u] = trA_lane_off<D>(lane, 32 * db, u);
  auto roff = [&](int s) __attribute__((always_inline)) { return roff_[s % KP] + (s / KP) * (16 * KP); };
  auto toff = [&](int db, int u) __attribute__((always_inline)) { return toff_[db % DP][u] + (db / DP) * (32 * DP); };

  if (ntiles > 0) issue_tile(0, 0);
  wait_vmem();
  __syncthreads();

  // One key tile; BUF (the LDS buffer holding it) is a compile-time
  // constant so that every LDS read is a lane register plus an immediate.
  auto tile = [&](auto bufc, int i) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    if (i + 1 < ntiles) issue_tile(i + 1, BUF ^ 1);
    const uint16_t* Ks = smem + BUF * C::BUF;
    const uint16_t* Vs = Ks + Tile::ELEMS;

    if (wave_active) {
      const bool second = i >= n0;
      const int k0 = (second ? seg.begin1 + (i - n0) : seg.begin0 + i) * BN;
      // At D >= 192 the intervals of the tile's half are derived from the
      // rows' blocks: selected from the two halves' copies, they ended up
      // read through a table of addresses in scratch memory.
      int lf, hf, ll, hl, lo, hi;
      if constexpr (ROW_BLOCKS) {
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
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int c0 = k0 + 32 * kb;
        if (c0 >= hl || c0 + 32 <= lf) continue;
        const bool full = ll <= c0 && c0 + 32 <= hf;
        // S^T and dP^T, two interleaved chains with the operand reads PF
        // products ahead (order pinned with scheduling barriers)
        constexpr int PF = 2;
        floatx16 sp = zero16(), dp = zero16();
        bf16x8 ak[C::KS], av[C::KS];
#pragma unroll
        for (int s = 0; s < PF; ++s) {
          ak[s] = lds_vec_at(Ks + 32 * kb * D + roff(s));
          av[s] = lds_vec_at(Vs + 32 * kb * D + roff(s));
        }
        mfma_burst_begin();
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          if (s + PF < C::KS) {
            ak[s + PF] = lds_vec_at(Ks + 32 * kb * D + roff(s + PF));
            av[s + PF] = lds_vec_at(Vs + 32 * kb * D + roff(s + PF));
          }
          sp = mfma32(ak[s], qf[s], sp);
          dp = mfma32(av[s], gf[s], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_burst_end();
        // P^T = exp2(S^T * scale * log2 e - LSE * log2 e), dS^T = P^T (dP^T - delta)
        if constexpr (SC) {
          // sp becomes P (1 - tanh^2): all that dS needs
          const Softcap capc = softcap_consts(a.scale, a.softcap);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float rr = softcap_r(capc, sp[r]);
            sp[r] = fast_exp2(softcap_y(capc, rr) - lse2) * (4.f * rr * (1.f - rr));
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sp[r] = fast_exp2(__builtin_fmaf(sp[r], a.scale_log2, -lse2));
        }
        if (!full) {
          // register r holds key c0 + 8 (r / 4) + 4 h2 + r % 4
          const int rl = lo - c0 - 4 * h2, rh = hi - c0 - 4 * h2;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            sp[r] = (off >= rl && off < rh) ? sp[r] : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = sp[r] * (dp[r] + ndlt);
        const bf16x8 sb0 = pack_bf16x8(dp, 0), sb1 = pack_bf16x8(dp, 8);
        // dQ^T += K^T dS^T
        mfma_burst_begin();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint16_t* kr = Ks + (32 * kb + 16 * ks) * D;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            dq[db] = mfma32(lds_trA_at(kr + toff(db, 0), kr + toff(db, 1)), ks ? sb1 : sb0, dq[db]);
        }
        mfma_burst_end();
      }
    }

    wait_vmem();
    __syncthreads();
  };

  for (int i = 0; i < ntiles; i += 2) {
    tile(std::integral_constant<int, 0>{}, i);
    if (i + 1 < ntiles) tile(std::integral_constant<int, 1>{}, i + 1);
  }

  if (wave_active && p < n) {
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

template <int D, bool GROUPED>
static void launch_dkdv(const AttnArgs& a, bool diag, hipStream_t s) {
  using KC = DkdvCfg<D, false, GROUPED>;
  const int ktiles = (a.n + KC::BKV - 1) / KC::BKV;
  const long long kblocks = (long long)ktiles * (diag ? 1 : a.nhalves) * a.B * a.Hkv * a.S;
  const dim3 grid((unsigned)kblocks), block(KC::NT);
  if (a.softcap > 0.f)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, GROUPED, true>), grid, block, 0, s, a, ktiles);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, GROUPED, false>), grid, block, 0, s, a, ktiles);
}

template <int D>
static hipError_t launch_stage_t(const AttnArgs& a, int stage, hipStream_t s) {
  if (stage == 0) {
    using QC = DqCfg<D>;
    const int qtiles = (a.n + QC::BM - 1) / QC::BM;
    const long long qblocks = (long long)qtiles * a.nhalves * a.B * a.H;
    if (a.softcap > 0.f)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)qblocks), dim3(QC::NT), 0, s, a, qtiles);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)qblocks), dim3(QC::NT), 0, s, a, qtiles);
  } else {
    // with the noisy-diagonal kernel the main grid holds the clean key tiles
    // only (they come first in its order)
    const bool diag = use_noisy_diag(a.mode, a.b);
    if (a.G > 1)
      launch_dkdv<D, true>(a, diag, s);
    else
      launch_dkdv<D, false>(a, diag, s);
    if (a.S > 1) {
      const long long E = a.tokens * a.Hkv * D;
      const long long rblocks = (2 * E / 8 + 255) / 256;
      hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)rblocks), dim3(256), 0, s, a.part, a.dk,
                         a.dv, E, a.S, a.cu, a.B, a.Hkv * D, diag ? 1 : 0, a.T);
    }
#ifdef BDATTN_NOISY_DIAG_KERNEL
    if (diag) {
      using DC = DiagCfg<D>;
      const int dtiles = (a.n + DC::BKV - 1) / DC::BKV;
      const dim3 dgrid((unsigned)((long long)dtiles * a.B * a.Hkv)), dblock(DC::NT);
      if (a.softcap > 0.f) {
        if (a.G > 1)
          hipLaunchKernelGGL((bwd_noisy_diag_kernel<D, true, true>), dgrid, dblock, 0, s, a, dtiles);
        else
          hipLaunchKernelGGL((bwd_noisy_diag_kernel<D, false, true>), dgrid, dblock, 0, s, a, dtiles);
      } else {
        if (a.G > 1)
          hipLaunchKernelGGL((bwd_noisy_diag_kernel<D, true, false>), dgrid, dblock, 0, s, a, dtiles);
        else
          hipLaunchKernelGGL((bwd_noisy_diag_kernel<D, false, false>), dgrid, dblock, 0, s, a, dtiles);
      }
    }
#endif
  }
  return hipGetLastError();
}

// Fewer dK/dV workgroups than four per resident slot (256 CUs times the
// workgroups one CU holds) leave CUs idle or the tail unbalanced.  The
// count follows the uncapped instances (the softcapped D = 96 one holds one
// workgroup per CU, not two), so that the workspace size does not depend on
// the cap.
constexpr long long kDkdvMinBlocksPerSlot = 4 * 256;

template <int D>
constexpr long long dkdv_min_blocks() {
  return kDkdvMinBlocksPerSlot * DkdvCfg<D, false, true>::WGS;
}

// Only grouped heads split (G = 1 gives S = 1), so the grouped tile sizes
// decide.
int dkdv_group_splits(int B, int n, int nhalves, int Hkv, int G, int D) {
  const int bkv = D == 64    ? DkdvCfg<64, false, true>::BKV
                  : D == 96  ? DkdvCfg<96, false, true>::BKV
                  : D == 128 ? DkdvCfg<128, false, true>::BKV
                  : D == 192 ? DkdvCfg<192, false, true>::BKV
                             : DkdvCfg<256, false, true>::BKV;
  const long long min_blocks = D == 64    ? dkdv_min_blocks<64>()
                               : D == 96  ? dkdv_min_blocks<96>()
                               : D == 128 ? dkdv_min_blocks<128>()
                               : D == 192 ? dkdv_min_blocks<192>()
                                          : dkdv_min_blocks<256>();
  const long long ktiles = ((long long)n + bkv - 1) / bkv;
  const long long base = ktiles * nhalves * B * Hkv;
  int S = 1;
  for (int c = 1; c <= G; ++c) {
    if (G % c) continue;
    S = c;
    if (base * c >= min_blocks) break;
  }
  return S;
}

hipError_t launch_bwd_stage(const AttnArgs& a, int D, int stage, hipStream_t s) {
  if (D == 64) return launch_stage_t<64>(a, stage, s);
  if (D == 96) return launch_stage_t<96>(a, stage, s);
  if (D == 192) return launch_stage_t<192>(a, stage, s);
  if (D == 256) return launch_stage_t<256>(a, stage, s);
  return launch_stage_t<128>(a, stage, s);
}

hipError_t launch_bwd(const AttnArgs& a, int D, hipStream_t s) {
  for (int stage = 0; stage < 2; ++stage) {
    hipError_t e = launch_bwd_stage(a, D, stage, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bd
