// api.cpp -- the extern "C" entry points declared in include/bdattn.h.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime; on error it returns a status code and launches nothing.  The
// library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "bdattn.h"
#include "geometry.h"
#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Limits of one [B][T][H][D] tensor.  Offsets are 64-bit, but grid sizes
// are 32-bit: the attention grids have at most ceil(T / 64) * B * H blocks.
// B * T * H rows are capped at 2^31 - 1 (512 GB of bf16 at D = 128, more
// than a GPU holds) so that any per-row count fits a 32-bit int.
int check_shape(int B, int T, int H, int D) {
  if (B < 1 || T < 1 || H < 1) return BDATTN_ERR_INVALID;
  if (D != 64 && D != 128) return BDATTN_ERR_UNSUPPORTED;
  const long long tiles = ((long long)T + 63) / 64 * B * H;
  if (tiles > (long long)std::numeric_limits<int>::max()) return BDATTN_ERR_INVALID;
  const long long rows = (long long)B * T * H;
  if (rows > (long long)std::numeric_limits<int>::max()) return BDATTN_ERR_INVALID;
  // The kernels address one half of one sample (all heads) through a 32-bit
  // buffer range: T/2 (or T) tokens x H x D bf16 must stay below 2 GiB.
  if ((long long)T * H * D * 2 >= (1LL << 31)) return BDATTN_ERR_UNSUPPORTED;
  return BDATTN_OK;
}

int check_scale(float scale) {
  return (std::isfinite(scale) && scale != 0.f) ? BDATTN_OK : BDATTN_ERR_INVALID;
}

// Grouped heads: 1 <= H_kv <= H and H a multiple of H_kv.
int check_kv_heads(int H, int H_kv) {
  return (H_kv >= 1 && H_kv <= H && H % H_kv == 0) ? BDATTN_OK : BDATTN_ERR_INVALID;
}

bd::AttnArgs make_args(int mode, int B, int n, int H, int H_kv, int b, float scale) {
  bd::AttnArgs a{};
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.G = H / H_kv;
  a.n = n;
  a.b = (mode == bd::MODE_CAUSAL) ? 1 : b;
  a.mode = mode;
  a.T = (mode == bd::MODE_CAUSAL) ? n : 2 * n;
  a.nhalves = (mode == bd::MODE_CAUSAL) ? 1 : 2;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

int fwd_common(int mode, const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int n, int H, int H_kv, int D, int b, float scale, void* stream) {
  if (!q || !k || !v || !out || !lse) return BDATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return BDATTN_ERR_INVALID;
  if (n < 1 || b < 1) return BDATTN_ERR_INVALID;
  if (mode == bd::MODE_DIFFUSION && n > std::numeric_limits<int>::max() / 2) return BDATTN_ERR_INVALID;
  int st = check_shape(B, mode == bd::MODE_CAUSAL ? n : 2 * n, H, D);
  if (st != BDATTN_OK) return st;
  if ((st = check_kv_heads(H, H_kv)) != BDATTN_OK) return st;
  if ((st = check_scale(scale)) != BDATTN_OK) return st;
  bd::AttnArgs a = make_args(mode, B, n, H, H_kv, b, scale);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  hipError_t e = bd::launch_fwd(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? BDATTN_OK : BDATTN_ERR_LAUNCH;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Backward workspace: -delta and lse2 per query row ([B][H][T] float32
// each), then, when the dK/dV kernel splits the groups of query heads
// (S > 1), float32 partial dK and dV ([S][B][T][H_kv][D] each).
size_t stats_bytes(int B, int T, int H) { return round256(2 * (size_t)B * H * T * sizeof(float)); }

int splits_of(int mode, int B, int n, int H, int H_kv) {
  return bd::dkdv_group_splits(B, n, mode == bd::MODE_CAUSAL ? 1 : 2, H_kv, H / H_kv);
}

size_t workspace_bytes(int mode, int B, int n, int H, int H_kv, int D) {
  if (n < 1 || (mode == bd::MODE_DIFFUSION && n > std::numeric_limits<int>::max() / 2)) return 0;
  const int T = (mode == bd::MODE_CAUSAL) ? n : 2 * n;
  if (check_shape(B, T, H, D) != BDATTN_OK || check_kv_heads(H, H_kv) != BDATTN_OK) return 0;
  const int S = splits_of(mode, B, n, H, H_kv);
  const size_t part = S > 1 ? 2 * (size_t)S * B * T * H_kv * D * sizeof(float) : 0;
  return stats_bytes(B, T, H) + round256(part);
}

int bwd_common(int mode, int stage, const void* q, const void* k, const void* v, const void* out,
               const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int n,
               int H, int H_kv, int D, int b, float scale, void* workspace, size_t ws_bytes,
               void* stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace)
    return BDATTN_ERR_INVALID;
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BDATTN_ERR_INVALID;
  if (n < 1 || b < 1) return BDATTN_ERR_INVALID;
  if (mode == bd::MODE_DIFFUSION && n > std::numeric_limits<int>::max() / 2) return BDATTN_ERR_INVALID;
  const int T = (mode == bd::MODE_CAUSAL) ? n : 2 * n;
  int st = check_shape(B, T, H, D);
  if (st != BDATTN_OK) return st;
  if ((st = check_kv_heads(H, H_kv)) != BDATTN_OK) return st;
  if ((st = check_scale(scale)) != BDATTN_OK) return st;
  if (ws_bytes < workspace_bytes(mode, B, n, H, H_kv, D)) return BDATTN_ERR_INVALID;
  bd::AttnArgs a = make_args(mode, B, n, H, H_kv, b, scale);
  a.S = splits_of(mode, B, n, H, H_kv);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse_in = lse;
  a.ndelta = static_cast<float*>(workspace);
  a.lse2 = a.ndelta + (size_t)B * H * T;
  a.part = a.S > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + stats_bytes(B, T, H))
                   : nullptr;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  hipError_t e = (stage < 0) ? bd::launch_bwd(a, D, static_cast<hipStream_t>(stream))
                             : bd::launch_bwd_stage(a, D, stage, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? BDATTN_OK : BDATTN_ERR_LAUNCH;
}

bool geom_args_ok(int mode, int n, int b) {
  return (mode == bd::MODE_DIFFUSION || mode == bd::MODE_CAUSAL) && n >= 1 && b >= 1;
}

}  // namespace

extern "C" {

const char* bdattn_status_string(int status) {
  switch (status) {
    case BDATTN_OK: return "ok";
    case BDATTN_ERR_INVALID: return "invalid argument";
    case BDATTN_ERR_UNSUPPORTED: return "unsupported head dimension (need 64 or 128)";
    case BDATTN_ERR_LAUNCH: return "HIP launch error";
    default: return "unknown status";
  }
}

int diffusion_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int n, int H, int D, int block_size, float scale, void* stream) {
  return fwd_common(bd::MODE_DIFFUSION, q, k, v, out, lse, B, n, H, H, D, block_size, scale,
                    stream);
}

int diffusion_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* stream) {
  return fwd_common(bd::MODE_DIFFUSION, q, k, v, out, lse, B, n, H, H_kv, D, block_size, scale,
                    stream);
}

size_t diffusion_attn_bwd_workspace_size(int B, int n, int H, int D) {
  return workspace_bytes(bd::MODE_DIFFUSION, B, n, H, H, D);
}

size_t diffusion_attn_bwd_gqa_workspace_size(int B, int n, int H, int H_kv, int D) {
  return workspace_bytes(bd::MODE_DIFFUSION, B, n, H, H_kv, D);
}

int diffusion_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int n, int H, int D, int block_size, float scale, void* workspace,
                       size_t workspace_bytes_, void* stream) {
  return bwd_common(bd::MODE_DIFFUSION, -1, q, k, v, out, dout, lse, dq, dk, dv, B, n, H, H, D,
                    block_size, scale, workspace, workspace_bytes_, stream);
}

int diffusion_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                           int n, int H, int H_kv, int D, int block_size, float scale,
                           void* workspace, size_t workspace_bytes_, void* stream) {
  return bwd_common(bd::MODE_DIFFUSION, -1, q, k, v, out, dout, lse, dq, dk, dv, B, n, H, H_kv, D,
                    block_size, scale, workspace, workspace_bytes_, stream);
}

int causal_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int S, int H, int D, float scale, void* stream) {
  return fwd_common(bd::MODE_CAUSAL, q, k, v, out, lse, B, S, H, H, D, 1, scale, stream);
}

int causal_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                        int S, int H, int H_kv, int D, float scale, void* stream) {
  return fwd_common(bd::MODE_CAUSAL, q, k, v, out, lse, B, S, H, H_kv, D, 1, scale, stream);
}

size_t causal_attn_bwd_workspace_size(int B, int S, int H, int D) {
  return workspace_bytes(bd::MODE_CAUSAL, B, S, H, H, D);
}

size_t causal_attn_bwd_gqa_workspace_size(int B, int S, int H, int H_kv, int D) {
  return workspace_bytes(bd::MODE_CAUSAL, B, S, H, H_kv, D);
}

int causal_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int S,
                    int H, int D, float scale, void* workspace, size_t workspace_bytes_,
                    void* stream) {
  return bwd_common(bd::MODE_CAUSAL, -1, q, k, v, out, dout, lse, dq, dk, dv, B, S, H, H, D, 1,
                    scale, workspace, workspace_bytes_, stream);
}

int causal_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int S, int H, int H_kv, int D, float scale, void* workspace,
                        size_t workspace_bytes_, void* stream) {
  return bwd_common(bd::MODE_CAUSAL, -1, q, k, v, out, dout, lse, dq, dk, dv, B, S, H, H_kv, D, 1,
                    scale, workspace, workspace_bytes_, stream);
}

int bdattn_bwd_stage(int mode, int stage, const void* q, const void* k, const void* v,
                     const void* out, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, int B, int n, int H, int H_kv, int D, int block_size, float scale,
                     void* workspace, size_t workspace_bytes_, void* stream) {
  if (mode != bd::MODE_DIFFUSION && mode != bd::MODE_CAUSAL) return BDATTN_ERR_INVALID;
  if (stage < 0 || stage > 1) return BDATTN_ERR_INVALID;
  return bwd_common(mode, stage, q, k, v, out, dout, lse, dq, dk, dv, B, n, H, H_kv, D,
                    mode == bd::MODE_CAUSAL ? 1 : block_size, scale, workspace, workspace_bytes_,
                    stream);
}

static int list_tiles(bool fwd, int mode, int n, int block_size, int tile_m, int tile_n, int half,
                      int tile, int32_t* entries, int max_entries) {
  if (!geom_args_ok(mode, n, block_size) || tile_m < 1 || tile_n < 1) return -1;
  if (max_entries > 0 && !entries) return -1;
  if (mode == bd::MODE_CAUSAL && half != bd::CLEAN) return -1;
  if (half != bd::NOISY && half != bd::CLEAN) return -1;
  const int own = fwd ? tile_m : tile_n;
  if (tile < 0 || (long long)tile * own >= n) return -1;
  const bd::Geom g{n, mode == bd::MODE_CAUSAL ? 1 : block_size};
  const bd::Segments s = fwd ? bd::fwd_segments(g, mode, half, tile, tile_m, tile_n)
                             : bd::bwd_segments(g, mode, half, tile, tile_m, tile_n);
  int count = 0;
  for (int i = 0; i < s.count; ++i) {
    for (int t = s.begin(i); t < s.end(i); ++t) {
      int r0, r1, c0, c1, qh, kh;
      if (fwd) {
        qh = half; kh = s.half(i);
        r0 = tile * tile_m; c0 = t * tile_n;
      } else {
        qh = s.half(i); kh = half;
        r0 = t * tile_m; c0 = tile * tile_n;
      }
      r1 = (tile_m >= n - r0) ? n : r0 + tile_m;
      c1 = (tile_n >= n - c0) ? n : c0 + tile_n;
      const int cls = bd::classify(g, qh, kh, r0, r1, c0, c1);
      if (cls == bd::TILE_SKIP) continue;
      if (count < max_entries) {
        entries[3 * count + 0] = s.half(i);
        entries[3 * count + 1] = t;
        entries[3 * count + 2] = cls == bd::TILE_PARTIAL ? 1 : 0;
      }
      ++count;
    }
  }
  return count;
}

int bdattn_fwd_tiles(int mode, int n, int block_size, int tile_m, int tile_n, int qhalf, int qt,
                     int32_t* entries, int max_entries) {
  return list_tiles(true, mode, n, block_size, tile_m, tile_n, qhalf, qt, entries, max_entries);
}

int bdattn_bwd_tiles(int mode, int n, int block_size, int tile_m, int tile_n, int khalf, int kt,
                     int32_t* entries, int max_entries) {
  return list_tiles(false, mode, n, block_size, tile_m, tile_n, khalf, kt, entries, max_entries);
}

int bdattn_row_interval(int mode, int n, int block_size, int qhalf, int p, int khalf, int32_t* lo,
                        int32_t* hi) {
  if (!geom_args_ok(mode, n, block_size) || !lo || !hi || p < 0 || p >= n) return -1;
  if (qhalf != bd::NOISY && qhalf != bd::CLEAN) return -1;
  if (khalf != bd::NOISY && khalf != bd::CLEAN) return -1;
  if (mode == bd::MODE_CAUSAL && (qhalf != bd::CLEAN || khalf != bd::CLEAN)) return -1;
  const bd::Geom g{n, mode == bd::MODE_CAUSAL ? 1 : block_size};
  int l, h;
  bd::row_interval(g, qhalf, khalf, p, l, h);
  *lo = l;
  *hi = h;
  return 0;
}

int64_t bdattn_visible_pairs(int mode, int n, int block_size) {
  if (!geom_args_ok(mode, n, block_size)) return -1;
  const bd::Geom g{n, mode == bd::MODE_CAUSAL ? 1 : block_size};
  int64_t total = 0;
  const int qhs[2] = {bd::NOISY, bd::CLEAN};
  for (int qi = 0; qi < 2; ++qi) {
    if (mode == bd::MODE_CAUSAL && qhs[qi] != bd::CLEAN) continue;
    for (int kh = 0; kh < 2; ++kh) {
      if (mode == bd::MODE_CAUSAL && kh != bd::CLEAN) continue;
      for (int p = 0; p < n; ++p) {
        int l, h;
        bd::row_interval(g, qhs[qi], kh, p, l, h);
        total += h - l;
      }
    }
  }
  return total;
}

}  // extern "C"
