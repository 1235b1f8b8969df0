// api.cpp -- the extern "C" entry points declared in include/bdattn.h.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime; on error it returns a status code and launches nothing.  The
// library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "bdattn.h"
#include "geometry.h"
#include "kernels.h"

namespace {

bool aligned(const void* p, unsigned bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// One call's problem.  Batched: B samples of T tokens (T = 2n, or n in
// causal mode).  Packed: B samples at the token offsets cu (device memory),
// `total` tokens in all, n the longest sample's half length (or length).
struct Problem {
  int mode;
  int B, n, H, Hkv, D, b;
  float scale;
  const int32_t* cu;  // packed only
  int total;          // packed only
  float softcap;      // > 0: scores capped to softcap * tanh(s / softcap); 0: off
  bool packed() const { return cu != nullptr; }
  int T() const { return mode == bd::MODE_CAUSAL ? n : 2 * n; }
  long long tokens() const { return packed() ? (long long)total : (long long)B * T(); }
};

// Shape limits.  Offsets are 64-bit, grid sizes 32-bit: the attention grids
// have at most ceil(T / 64) * B * H blocks.  All rows (tokens x H) are
// capped at 2^31 - 1 (512 GB of bf16 at D = 128, more than a GPU holds) so
// that any per-row count fits a 32-bit int.  The kernels address one half
// of one sample (all heads) through a 32-bit buffer range, so T / 2 (or T)
// tokens x H x D bf16 must stay below 2 GiB.
int check_problem(const Problem& p) {
  if (p.mode != bd::MODE_DIFFUSION && p.mode != bd::MODE_CAUSAL) return BDATTN_ERR_INVALID;
  if (p.B < 1 || p.n < 1 || p.H < 1 || p.b < 1) return BDATTN_ERR_INVALID;
  if (p.mode == bd::MODE_DIFFUSION && p.n > std::numeric_limits<int>::max() / 2)
    return BDATTN_ERR_INVALID;
  if (p.D != 64 && p.D != 96 && p.D != 128 && p.D != 192 && p.D != 256) return BDATTN_ERR_UNSUPPORTED;
  if (p.Hkv < 1 || p.Hkv > p.H || p.H % p.Hkv != 0) return BDATTN_ERR_INVALID;
  if (p.packed() && (p.total < 1 || !aligned(p.cu, 4))) return BDATTN_ERR_INVALID;
  const long long T = p.T();
  const long long tiles = (T + 63) / 64 * p.B * p.H;
  if (tiles > (long long)std::numeric_limits<int>::max()) return BDATTN_ERR_INVALID;
  if (p.tokens() * p.H > (long long)std::numeric_limits<int>::max()) return BDATTN_ERR_INVALID;
  if (T * p.H * p.D * 2 >= (1LL << 31)) return BDATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(p.scale) || p.scale == 0.f) return BDATTN_ERR_INVALID;
  if (!std::isfinite(p.softcap) || p.softcap < 0.f) return BDATTN_ERR_INVALID;
  return BDATTN_OK;
}

int splits_of(const Problem& p) {
  return bd::dkdv_group_splits(p.B, p.n, p.mode == bd::MODE_CAUSAL ? 1 : 2, p.Hkv, p.H / p.Hkv, p.D);
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Backward workspace: -delta and lse2 per query row ([B][H][T], or
// [H][total] packed, float32 each), then, when the dK/dV kernel splits the
// groups of query heads (S > 1), float32 partial dK and dV
// ([S][tokens][Hkv][D] each).
size_t stats_bytes(const Problem& p) {
  return round256(2 * (size_t)p.tokens() * p.H * sizeof(float));
}

size_t workspace_bytes(const Problem& p) {
  if (check_problem(p) != BDATTN_OK) return 0;
  const int S = splits_of(p);
  const size_t part = S > 1 ? 2 * (size_t)S * p.tokens() * p.Hkv * p.D * sizeof(float) : 0;
  return stats_bytes(p) + round256(part);
}

bd::AttnArgs make_args(const Problem& p) {
  bd::AttnArgs a{};
  a.B = p.B;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.G = p.H / p.Hkv;
  a.S = 1;
  a.n = p.n;
  a.b = (p.mode == bd::MODE_CAUSAL) ? 1 : p.b;
  a.mode = p.mode;
  a.T = p.T();
  a.nhalves = (p.mode == bd::MODE_CAUSAL) ? 1 : 2;
  a.scale = p.scale;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.softcap = p.softcap;
  a.cu = p.cu;
  a.tokens = p.tokens();
  a.stat_hs = p.packed() ? p.total : p.T();
  return a;
}

int run_fwd(const Problem& p, const void* q, const void* k, const void* v, void* out, float* lse,
            void* stream) {
  if (!q || !k || !v || !out || !lse) return BDATTN_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 16))
    return BDATTN_ERR_INVALID;
  const int st = check_problem(p);
  if (st != BDATTN_OK) return st;
  bd::AttnArgs a = make_args(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  hipError_t e = bd::launch_fwd(a, p.D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? BDATTN_OK : BDATTN_ERR_LAUNCH;
}

int run_fwd_fp8(const Problem& p, const void* q, const void* k, const void* v, const float* qd,
                const float* kd, const float* vd, void* out, float* lse, void* stream) {
  if (!q || !k || !v || !qd || !kd || !vd || !out || !lse) return BDATTN_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 16))
    return BDATTN_ERR_INVALID;
  if (!aligned(qd, 4) || !aligned(kd, 4) || !aligned(vd, 4)) return BDATTN_ERR_INVALID;
  const int st = check_problem(p);
  if (st != BDATTN_OK) return st;
  if (p.D != 64 && p.D != 128) return BDATTN_ERR_UNSUPPORTED;  // the FP8 forward takes D = 64 or 128
  bd::AttnArgs a = make_args(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.qd = qd;
  a.kd = kd;
  a.vd = vd;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  hipError_t e = bd::launch_fwd_fp8(a, p.D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? BDATTN_OK : BDATTN_ERR_LAUNCH;
}

// stage < 0: the whole backward
int run_bwd(const Problem& p, int stage, const void* q, const void* k, const void* v,
            const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
            void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace)
    return BDATTN_ERR_INVALID;
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned(ptr, 16)) return BDATTN_ERR_INVALID;
  const int st = check_problem(p);
  if (st != BDATTN_OK) return st;
  if (ws_bytes < workspace_bytes(p)) return BDATTN_ERR_INVALID;
  bd::AttnArgs a = make_args(p);
  a.S = splits_of(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse_in = lse;
  a.ndelta = static_cast<float*>(workspace);
  a.lse2 = a.ndelta + (size_t)p.tokens() * p.H;
  a.part = a.S > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + stats_bytes(p))
                   : nullptr;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  hipError_t e = (stage < 0) ? bd::launch_bwd(a, p.D, static_cast<hipStream_t>(stream))
                             : bd::launch_bwd_stage(a, p.D, stage, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? BDATTN_OK : BDATTN_ERR_LAUNCH;
}

// ---- the static scratch of diffusion_attn_bwd_noalloc ----------------------
//
// For callers that cannot allocate: the backward's per-row statistics
// (-delta and lse2, 8 bytes per query row and head) live in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy (loaded with the code object) until the process ends.
// Host code never uses the array's name as an address: its device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The device the call's work runs on (the stream's, or the current one for
// the null stream) and that device's address of scratch.
int scratch_of(void* stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return BDATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return BDATTN_ERR_INVALID;
  if (dev < 0 || dev >= kMaxDevices) return BDATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return BDATTN_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return BDATTN_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return BDATTN_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return BDATTN_OK;
}

Problem batched(int mode, int B, int n, int H, int H_kv, int D, int b, float scale) {
  return Problem{mode, B, n, H, H_kv, D, mode == bd::MODE_CAUSAL ? 1 : b, scale, nullptr, 0, 0.f};
}

Problem packed(int mode, const int32_t* cu, int B, int max_n, int total, int H, int H_kv, int D,
               int b, float scale) {
  return Problem{mode, B, max_n, H, H_kv, D, mode == bd::MODE_CAUSAL ? 1 : b, scale, cu, total, 0.f};
}

// The general form: batched (cu NULL) or packed, either mode, with softcap.
Problem general(int mode, const int32_t* cu, int B, int n, int total, int H, int H_kv, int D, int b,
                float scale, float softcap) {
  Problem p = cu ? packed(mode, cu, B, n, total, H, H_kv, D, b, scale)
                 : batched(mode, B, n, H, H_kv, D, b, scale);
  p.softcap = softcap;
  return p;
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
    case BDATTN_ERR_UNSUPPORTED: return "unsupported head dimension (need 64, 96, 128, 192 or 256) or size";
    case BDATTN_ERR_LAUNCH: return "HIP launch error";
    case BDATTN_ERR_TOO_LARGE:
      return "problem needs more than the 32 MiB static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

// ---- batched, H_kv = H ----------------------------------------------------

int diffusion_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int n, int H, int D, int block_size, float scale, void* stream) {
  return run_fwd(batched(bd::MODE_DIFFUSION, B, n, H, H, D, block_size, scale), q, k, v, out, lse,
                 stream);
}

size_t diffusion_attn_bwd_workspace_size(int B, int n, int H, int D) {
  return workspace_bytes(batched(bd::MODE_DIFFUSION, B, n, H, H, D, 1, 1.f));
}

int diffusion_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int n, int H, int D, int block_size, float scale, void* workspace,
                       size_t workspace_bytes_, void* stream) {
  return run_bwd(batched(bd::MODE_DIFFUSION, B, n, H, H, D, block_size, scale), -1, q, k, v, out,
                 dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
}

int diffusion_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               int B, int n, int H, int D, int block_size, float scale,
                               void* stream) {
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (ptr == nullptr || !aligned(ptr, 16)) return BDATTN_ERR_INVALID;
  const Problem p = batched(bd::MODE_DIFFUSION, B, n, H, H, D, block_size, scale);
  const int st = check_problem(p);
  if (st != BDATTN_OK) return st;
  if (workspace_bytes(p) > kScratchBytes) return BDATTN_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int sst = scratch_of(stream, &ws);
  if (sst != BDATTN_OK) return sst;
  return run_bwd(p, -1, q, k, v, out, dout, lse, dq, dk, dv, ws, kScratchBytes, stream);
}

int causal_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int S, int H, int D, float scale, void* stream) {
  return run_fwd(batched(bd::MODE_CAUSAL, B, S, H, H, D, 1, scale), q, k, v, out, lse, stream);
}

size_t causal_attn_bwd_workspace_size(int B, int S, int H, int D) {
  return workspace_bytes(batched(bd::MODE_CAUSAL, B, S, H, H, D, 1, 1.f));
}

int causal_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int S,
                    int H, int D, float scale, void* workspace, size_t workspace_bytes_,
                    void* stream) {
  return run_bwd(batched(bd::MODE_CAUSAL, B, S, H, H, D, 1, scale), -1, q, k, v, out, dout, lse, dq,
                 dk, dv, workspace, workspace_bytes_, stream);
}

// ---- batched, grouped heads -----------------------------------------------

int diffusion_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* stream) {
  return run_fwd(batched(bd::MODE_DIFFUSION, B, n, H, H_kv, D, block_size, scale), q, k, v, out,
                 lse, stream);
}

size_t diffusion_attn_bwd_gqa_workspace_size(int B, int n, int H, int H_kv, int D) {
  return workspace_bytes(batched(bd::MODE_DIFFUSION, B, n, H, H_kv, D, 1, 1.f));
}

int diffusion_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                           int n, int H, int H_kv, int D, int block_size, float scale,
                           void* workspace, size_t workspace_bytes_, void* stream) {
  return run_bwd(batched(bd::MODE_DIFFUSION, B, n, H, H_kv, D, block_size, scale), -1, q, k, v,
                 out, dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
}

int causal_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                        int S, int H, int H_kv, int D, float scale, void* stream) {
  return run_fwd(batched(bd::MODE_CAUSAL, B, S, H, H_kv, D, 1, scale), q, k, v, out, lse, stream);
}

size_t causal_attn_bwd_gqa_workspace_size(int B, int S, int H, int H_kv, int D) {
  return workspace_bytes(batched(bd::MODE_CAUSAL, B, S, H, H_kv, D, 1, 1.f));
}

int causal_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int S, int H, int H_kv, int D, float scale, void* workspace,
                        size_t workspace_bytes_, void* stream) {
  return run_bwd(batched(bd::MODE_CAUSAL, B, S, H, H_kv, D, 1, scale), -1, q, k, v, out, dout, lse,
                 dq, dk, dv, workspace, workspace_bytes_, stream);
}

// ---- FP8 (E4M3) forward -------------------------------------------------------

int diffusion_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                           const float* k_descale, const float* v_descale, void* out, float* lse,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* stream) {
  return run_fwd_fp8(batched(bd::MODE_DIFFUSION, B, n, H, H_kv, D, block_size, scale), q, k, v,
                     q_descale, k_descale, v_descale, out, lse, stream);
}

int causal_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, const float* v_descale, void* out, float* lse,
                        int B, int S, int H, int H_kv, int D, float scale, void* stream) {
  return run_fwd_fp8(batched(bd::MODE_CAUSAL, B, S, H, H_kv, D, 1, scale), q, k, v, q_descale,
                     k_descale, v_descale, out, lse, stream);
}

// ---- packed variable-length samples -----------------------------------------
// total_tokens = 0: nothing to compute (BDATTN_OK, nothing launched).

int diffusion_attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              const int32_t* cu_seqlens, int B, int max_n, int total_tokens, int H,
                              int H_kv, int D, int block_size, float scale, void* stream) {
  if (total_tokens == 0) return BDATTN_OK;
  if (!cu_seqlens) return BDATTN_ERR_INVALID;
  return run_fwd(packed(bd::MODE_DIFFUSION, cu_seqlens, B, max_n, total_tokens, H, H_kv, D,
                        block_size, scale),
                 q, k, v, out, lse, stream);
}

size_t diffusion_attn_varlen_bwd_workspace_size(int B, int max_n, int total_tokens, int H, int H_kv,
                                                int D) {
  if (total_tokens == 0) return 0;
  // the offsets are not read here; any aligned non-null stand-in will do
  static const int32_t stand_in = 0;
  return workspace_bytes(packed(bd::MODE_DIFFUSION, &stand_in, B, max_n, total_tokens, H, H_kv, D,
                                1, 1.f));
}

int diffusion_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens, int B, int max_n, int total_tokens, int H,
                              int H_kv, int D, int block_size, float scale, void* workspace,
                              size_t workspace_bytes_, void* stream) {
  if (total_tokens == 0) return BDATTN_OK;
  if (!cu_seqlens) return BDATTN_ERR_INVALID;
  return run_bwd(packed(bd::MODE_DIFFUSION, cu_seqlens, B, max_n, total_tokens, H, H_kv, D,
                        block_size, scale),
                 -1, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
}

int causal_attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* cu_seqlens, int B, int max_S, int total_tokens, int H,
                           int H_kv, int D, float scale, void* stream) {
  if (total_tokens == 0) return BDATTN_OK;
  if (!cu_seqlens) return BDATTN_ERR_INVALID;
  return run_fwd(packed(bd::MODE_CAUSAL, cu_seqlens, B, max_S, total_tokens, H, H_kv, D, 1, scale),
                 q, k, v, out, lse, stream);
}

size_t causal_attn_varlen_bwd_workspace_size(int B, int max_S, int total_tokens, int H, int H_kv,
                                             int D) {
  if (total_tokens == 0) return 0;
  static const int32_t stand_in = 0;
  return workspace_bytes(packed(bd::MODE_CAUSAL, &stand_in, B, max_S, total_tokens, H, H_kv, D, 1,
                                1.f));
}

int causal_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           const int32_t* cu_seqlens, int B, int max_S, int total_tokens, int H,
                           int H_kv, int D, float scale, void* workspace, size_t workspace_bytes_,
                           void* stream) {
  if (total_tokens == 0) return BDATTN_OK;
  if (!cu_seqlens) return BDATTN_ERR_INVALID;
  return run_bwd(packed(bd::MODE_CAUSAL, cu_seqlens, B, max_S, total_tokens, H, H_kv, D, 1, scale),
                 -1, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
}

// ---- the general form ----------------------------------------------------------

int bdattn_fwd(int mode, const void* q, const void* k, const void* v, void* out, float* lse,
               const int32_t* cu_seqlens, int B, int n, int total_tokens, int H, int H_kv, int D,
               int block_size, float scale, float softcap, void* stream) {
  if (mode != bd::MODE_DIFFUSION && mode != bd::MODE_CAUSAL) return BDATTN_ERR_INVALID;
  if (cu_seqlens && total_tokens == 0) return BDATTN_OK;
  return run_fwd(general(mode, cu_seqlens, B, n, total_tokens, H, H_kv, D, block_size, scale, softcap),
                 q, k, v, out, lse, stream);
}

size_t bdattn_bwd_workspace_size(int mode, int packed_, int B, int n, int total_tokens, int H,
                                 int H_kv, int D) {
  if (mode != bd::MODE_DIFFUSION && mode != bd::MODE_CAUSAL) return 0;
  if (packed_ && total_tokens == 0) return 0;
  static const int32_t stand_in = 0;  // the offsets are not read here
  return workspace_bytes(general(mode, packed_ ? &stand_in : nullptr, B, n, total_tokens, H, H_kv, D,
                                 1, 1.f, 0.f));
}

int bdattn_bwd(int mode, const void* q, const void* k, const void* v, const void* out,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               const int32_t* cu_seqlens, int B, int n, int total_tokens, int H, int H_kv, int D,
               int block_size, float scale, float softcap, void* workspace,
               size_t workspace_bytes_, void* stream) {
  if (mode != bd::MODE_DIFFUSION && mode != bd::MODE_CAUSAL) return BDATTN_ERR_INVALID;
  if (cu_seqlens && total_tokens == 0) return BDATTN_OK;
  return run_bwd(general(mode, cu_seqlens, B, n, total_tokens, H, H_kv, D, block_size, scale, softcap),
                 -1, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
}

// ---- one backward stage -----------------------------------------------------

int bdattn_bwd_stage(int mode, int stage, const void* q, const void* k, const void* v,
                     const void* out, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, const int32_t* cu_seqlens, int B, int n, int total_tokens, int H,
                     int H_kv, int D, int block_size, float scale, float softcap, void* workspace,
                     size_t workspace_bytes_, void* stream) {
  if (mode != bd::MODE_DIFFUSION && mode != bd::MODE_CAUSAL) return BDATTN_ERR_INVALID;
  if (stage < 0 || stage > 1) return BDATTN_ERR_INVALID;
  if (cu_seqlens && total_tokens == 0) return BDATTN_OK;
  return run_bwd(general(mode, cu_seqlens, B, n, total_tokens, H, H_kv, D, block_size, scale, softcap),
                 stage, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes_, stream);
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
