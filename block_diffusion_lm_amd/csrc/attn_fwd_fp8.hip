// attn_fwd_fp8.hip -- forward pass on FP8 (OCP E4M3) inputs: O and the
// per-row log-sum-exp of softmax(scale * q.k under the mask) v, where q, k
// and v are E4M3 values times a float32 descale factor per (sample, head).
//
// Fast Diffusion Attention, "Results" (the FP8 forward pass).  The tile walk,
// masking and online softmax are those of the bf16 forward (attn_fwd.hip:
// FlashAttention sections 4.1, 4.2, 5.1; Fast Diffusion Attention "Visit
// only the visible tiles"), with two changes:
//  * both products run on v_mfma_f32_32x32x64 with E4M3 operands: S^T = K
//    Q^T contracts 64 head dimensions per instruction, O^T += V^T P^T all 64
//    keys of a tile;
//  * the unnormalised probabilities P~ = 2^(s c - m) (at most 2^8 under the
//    lazy rescale, inside E4M3's range of 448) are rounded to E4M3 for the
//    P.V product; the denominator sums the unrounded float32 values.  The
//    scores carry the factor scale * q_descale * k_descale, the output
//    v_descale / l.
//
// Operand layouts (both probed on the hardware): a lane l of a 32x32x64
// product holds row (or column) l % 32 and the 32 contraction indices
// [32 (l / 32), +32), as 32 bytes, in the same order for A and B.  S^T's
// D-layout gives lane l the 32 keys {32 kb + 8 g + 4 (l / 32) + i} of its
// query row; packed in register order they are P^T's B operand.  V's
// matching A operand comes from ds_read_b64_tr_b8 (each 16-lane group reads
// 8 rows x 16 columns of bytes, lane i receiving column i): V's rows are
// permuted as they are copied into LDS so that those reads return the keys
// in exactly that order.
#include "common.h"
#include "geometry.h"
#include "kernels.h"

#include <type_traits>

namespace bd {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// E4M3 tiles of [rows][D] bytes in LDS: 16-byte chunk c of row r sits at
// chunk c ^ swz8(r).  Free of bank conflicts (64 banks of 4 bytes) for the
// two reads below: 16 consecutive rows of one chunk (ds_read_b128, K as the
// A operand), and 8 rows x two adjacent chunks (the transposing reads of
// two 16-lane groups).
template <int D>
__device__ __forceinline__ int swz8(int r) {
  if constexpr (D == 128) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
  return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}

// LDS row rho of a V tile holds key vkey(rho): rho = 32 h + j carries the
// key of byte j of the P^T operand of lane half h.
__device__ __forceinline__ int vkey(int rho) {
  const int h = rho >> 5, j = rho & 31;
  return 32 * (j >> 4) + 8 * ((j >> 2) & 3) + 4 * h + (j & 3);
}

// BN rows of D bytes copied straight into LDS by NT threads (16 bytes each
// per instruction); PERMUTE stores key vkey(rho) in row rho.
template <int BN, int D, int NT, bool PERMUTE>
struct Fp8Tile {
  static constexpr int CH = D / 16;
  static constexpr int SLOTS = BN * CH;
  static constexpr int PER = SLOTS / NT;
  static constexpr int BYTES = BN * D;
  static_assert(SLOTS % NT == 0, "tile must split evenly over the threads");
  __device__ __forceinline__ static void load(rsrc_t src, uint32_t row_bytes, int row0, uint32_t lds, int tid) {
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = i * NT + tid;
      const int rho = slot / CH;
      const int c = (slot % CH) ^ swz8<D>(rho);
      const int row = PERMUTE ? vkey(rho) : rho;
      const uint32_t voff = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
      lds_direct16(src, lds + (uint32_t)(i * NT + wbase) * 16u, voff, (uint32_t)row0 * row_bytes);
    }
  }
};

template <int D>
struct FwdFp8Cfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int KB = BN / 32;  // 32-key blocks per tile
  static constexpr int K8 = D / 64;   // products over the head dimension
  static constexpr int DB = D / 32;
  using KTile = Fp8Tile<BN, D, NT, false>;
  using VTile = Fp8Tile<BN, D, NT, true>;
  static constexpr int BUF = 2 * BN * D;  // bytes: K then V
};

// The running maximum is raised lazily, as in the bf16 forward: P~ stays at
// most 2^8, inside E4M3's range (largest value 448).
constexpr float kFp8RescaleThreshold = 8.0f;

__device__ __forceinline__ floatx16 mfma_fp8(i32x8 a, i32x8 b, floatx16 c) {
  // operand formats 0 = E4M3; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(AttnArgs a, int qtiles) {
  using C = FwdFp8Cfg<D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::BUF];
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
  if (!sample_of(a, bi, sample0, n, stat0) || qt * C::BM >= n) return;
  const Geom g{n, a.b};

  // rows of E4M3 bytes: q with H heads, k and v with Hkv
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q);
  const uint8_t* k8 = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* v8 = reinterpret_cast<const uint8_t*>(a.v);
  const size_t rs = (size_t)a.H * D;
  const size_t rs_kv = (size_t)a.Hkv * D;
  const int qoff = (a.mode == MODE_DIFFUSION && qh == CLEAN) ? n : 0;
  const uint32_t q_row_bytes = (uint32_t)rs;
  const uint32_t kv_row_bytes = (uint32_t)rs_kv;

  const float qd = a.qd[(size_t)bi * a.H + hh];
  const float kd = a.kd[(size_t)bi * a.Hkv + hk];
  const float vd = a.vd[(size_t)bi * a.Hkv + hk];
  const float sfac = a.scale * qd * kd;  // multiplies the raw E4M3 scores

  const int q0 = qt * C::BM;
  const int pw0 = q0 + 32 * w;
  const int pw1 = min(pw0 + 32, n);
  const bool wave_active = pw0 < n;
  const int p = pw0 + l32;

  // Q^T operand: lane (row p, half h2) holds bytes [64 s + 32 h2, +32) of
  // its row; rows past the half read as zero.  A negative score factor is
  // folded into Q (the sign bit of every byte; exact).
  i32x8 qf[C::K8];
  {
    const rsrc_t rq = make_rsrc(q8 + (sample0 + qoff) * rs + (size_t)hh * D, (uint32_t)n * q_row_bytes);
    const uint32_t flip = sfac < 0.f ? 0x80808080u : 0u;
#pragma unroll
    for (int s = 0; s < C::K8; ++s) {
      const uint32_t off = (uint32_t)p * q_row_bytes + (uint32_t)(64 * s + 32 * h2);
      const u32x4 lo = buf_ld16(rq, off, 0) ^ flip;
      const u32x4 hi = buf_ld16(rq, off + 16u, 0) ^ flip;
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int s = 0; s < C::K8; ++s) settle(qf[s]);
  }
  const float cs = fabsf(sfac) * kLog2e;

  const Segments seg = fwd_segments(g, a.mode, qh, qt, C::BM, BN);
  const int n0 = seg.count > 0 ? seg.end0 - seg.begin0 : 0;
  const int ntiles = seg.tiles();

  // visible intervals of the wave's first, last and own rows per key half
  int lo_f0, hi_f0, lo_l0, hi_l0, lo_p0, hi_p0, lo_f1, hi_f1, lo_l1, hi_l1, lo_p1, hi_p1;
  row_interval(g, qh, seg.half0, pw0, lo_f0, hi_f0);
  row_interval(g, qh, seg.half0, max(pw1 - 1, pw0), lo_l0, hi_l0);
  row_interval(g, qh, seg.half0, p, lo_p0, hi_p0);
  row_interval(g, qh, seg.half1, pw0, lo_f1, hi_f1);
  row_interval(g, qh, seg.half1, max(pw1 - 1, pw0), lo_l1, hi_l1);
  row_interval(g, qh, seg.half1, p, lo_p1, hi_p1);
  auto kv_base = [&](int half) -> size_t {
    const int off = (a.mode == MODE_DIFFUSION && half == CLEAN) ? n : 0;
    return (sample0 + off) * rs_kv + (size_t)hk * D;
  };
  const size_t kvb0 = kv_base(seg.half0);
  const size_t kvb1 = kv_base(seg.half1);

  auto issue_tile = [&](int i, int buf) __attribute__((always_inline)) {
    const bool second = i >= n0;
    const int kt = second ? seg.begin1 + (i - n0) : seg.begin0 + i;
    const size_t kvb = second ? kvb1 : kvb0;
    const uint32_t dst = sbase + (uint32_t)(buf * C::BUF);
    const uint32_t bytes = (uint32_t)n * kv_row_bytes;
    C::KTile::load(make_rsrc(k8 + kvb, bytes), kv_row_bytes, kt * BN, dst, tid);
    C::VTile::load(make_rsrc(v8 + kvb, bytes), kv_row_bytes, kt * BN, dst + BN * D, tid);
  };

  floatx16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Per-lane LDS byte offsets: K rows (key l32 of a block, chunks 4s + 2h2
  // and the next) and the transposing reads of V (row 32 h2 + 8 t + s / 2,
  // byte column 32 db + 16 (group % 2) + 8 (s % 2)).
  int koff[C::K8][2];
#pragma unroll
  for (int s = 0; s < C::K8; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = 4 * s + 2 * h2 + u;
      koff[s][u] = l32 * D + ((c ^ swz8<D>(l32)) << 4);
    }
  int voff[C::DB][4];
  {
    const int sl = lane & 15, gc = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 32 * h2 + 8 * t + (sl >> 1);
        const int col = 32 * db + 16 * gc + 8 * (sl & 1);
        voff[db][t] = row * D + (((col >> 4) ^ swz8<D>(row)) << 4) + (col & 15);
      }
  }

  if (ntiles > 0) issue_tile(0, 0);
  wait_vmem();
  __syncthreads();

  auto tile = [&](auto bufc, int i) __attribute__((always_inline)) {
    constexpr int BUFI = decltype(bufc)::value;
    if (i + 1 < ntiles) issue_tile(i + 1, BUFI ^ 1);
    const uint8_t* Ks = smem + BUFI * C::BUF;
    const uint8_t* Vs = Ks + BN * D;

    if (wave_active) {
      const bool second = i >= n0;
      const int k0 = (second ? seg.begin1 + (i - n0) : seg.begin0 + i) * BN;
      const int lf = second ? lo_f1 : lo_f0, hf = second ? hi_f1 : hi_f0;
      const int ll = second ? lo_l1 : lo_l0, hl = second ? hi_l1 : hi_l0;
      const int lo = second ? lo_p1 : lo_p0, hi = second ? hi_p1 : hi_p0;
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
        const uint8_t* kr = Ks + 32 * kb * D;
#pragma unroll
        for (int s = 0; s < C::K8; ++s) {
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(kr + koff[s][0]);
          const u32x4 x1 = *reinterpret_cast<const u32x4*>(kr + koff[s][1]);
          const i32x8 ka = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                            (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          acc = mfma_fp8(ka, qf[s], acc);
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
      const float m_tile = halves_max(mt) * cs;
      const float m_cand = fmaxf(m_run, m_tile);
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kFp8RescaleThreshold)) {
        const float alpha = (m_cand > m_run) ? fast_exp2(m_run - m_cand) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_cand;
      }
      const float nbase = (m_run == -INFINITY) ? 0.f : -m_run;

      if (cls[0] != TILE_SKIP || cls[1] != TILE_SKIP) {
        // P^T as E4M3 bytes in register order: dword 4 kb + u holds
        // registers 4u .. 4u + 3 of block kb; a skipped block is zero
        i32x8 pf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          if (cls[kb] == TILE_SKIP) {
#pragma unroll
            for (int u = 0; u < 4; ++u) pf[4 * kb + u] = 0;
            continue;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(__builtin_fmaf(sc[kb][r], cs, nbase));
            sc[kb][r] = pr;
            l_run += pr;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(sc[kb][4 * u], sc[kb][4 * u + 1], 0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(sc[kb][4 * u + 2], sc[kb][4 * u + 3], wd, true);
            pf[4 * kb + u] = wd;
          }
        }
        // O^T += V^T P^T over all 64 keys of the tile
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          i32x8 va;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(Vs + voff[db][t]));
            va[2 * t] = x[0];
            va[2 * t + 1] = x[1];
          }
          o[db] = mfma_fp8(va, pf, o[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };

  for (int i = 0; i < ntiles; i += 2) {
    tile(std::integral_constant<int, 0>{}, i);
    if (i + 1 < ntiles) tile(std::integral_constant<int, 1>{}, i + 1);
  }

  // Epilogue: O = z * v_descale / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = halves_sum(l_run);
  if (wave_active && p < n) {
    const float f = vd / l_tot;
    uint16_t* orow = a.out + (sample0 + qoff + p) * rs + (size_t)hh * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * h2;
        u32x2 pk = {pack2_bf16(o[db][4 * gq] * f, o[db][4 * gq + 1] * f),
                    pack2_bf16(o[db][4 * gq + 2] * f, o[db][4 * gq + 3] * f)};
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
    if (h2 == 0)
      a.lse[stat0 + (size_t)hh * a.stat_hs + qoff + p] = (m_run + log2f(l_tot)) * kLn2;
  }
}

hipError_t launch_fwd_fp8(const AttnArgs& a, int D, hipStream_t s) {
  using C = FwdFp8Cfg<128>;
  static_assert(FwdFp8Cfg<64>::BM == C::BM, "one query tile size for both widths");
  const int qtiles = (a.n + C::BM - 1) / C::BM;
  const long long blocks = (long long)qtiles * a.nhalves * a.B * a.H;
  if (D == 64)
    hipLaunchKernelGGL((fwd_fp8_kernel<64>), dim3((unsigned)blocks), dim3(C::NT), 0, s, a, qtiles);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<128>), dim3((unsigned)blocks), dim3(C::NT), 0, s, a, qtiles);
  return hipGetLastError();
}

}  // namespace bd
