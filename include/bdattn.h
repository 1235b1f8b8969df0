/*
 * bdattn.h -- C ABI of the block-diffusion attention library (libbdattn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (Fast Diffusion Attention, sections "TL;DR" and "Block
 * diffusion in one picture"): exact softmax attention over a sequence of 2n
 * tokens laid out as [noisy | clean], under the block-diffusion mask of
 * block size b.  Blocks are consecutive runs of b tokens from the start of
 * each half (the last block of a half is shorter when b does not divide n).
 * A noisy block attends to itself in both directions and to every clean
 * block strictly before it; a clean block attends to itself and to the
 * clean blocks before it; every other (query, key) pair is masked.
 *
 * The causal entry points compute top-left causal attention (query i sees
 * keys 0..i of its own sequence) with the same tile engine.  Viewing a
 * [B, 2n, H, D] tensor as [2B, n, H, D] gives the equal-work yardstick of
 * "The right yardstick" section.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are caller-owned device memory, contiguous, 16-byte aligned.
 *    q, k, v, out, dout, dq, dk, dv: bfloat16, layout [B][T][H][D] with
 *    T = 2n (diffusion) or S (causal); the last dimension is contiguous.
 *  - lse: float32, layout [B][H][T]: the natural-log log-sum-exp of each
 *    query row's scaled scores (FlashAttention: Exact Attention Without
 *    Materialization, section 4.5: the statistic saved for the backward).
 *  - scale multiplies q.k before the softmax (callers usually pass
 *    1/sqrt(D)).  It must be finite and nonzero.
 *  - D must be 64, 96, 128, 192 or 256 (the FP8 forward: 64 or 128).
 *    B, n (or S), H >= 1.  block_size >= 1; a block longer than a half is
 *    allowed (one block per half).  One sample's
 *    tensor (2n or S tokens x H x D bf16) must be smaller than 2 GiB
 *    (BDATTN_ERR_UNSUPPORTED otherwise).
 *  - stream is a hipStream_t (NULL: the default stream).  Every call is
 *    asynchronous on that stream; faults during execution surface at the
 *    caller's next synchronisation.
 *  - Arguments are validated before anything is launched; on error nothing
 *    is written and nothing is launched.  The library allocates no memory
 *    and keeps no state between calls, so calls are reentrant; the one
 *    exception is diffusion_attn_bwd_noalloc, whose calls share a static
 *    device array per GPU (see there).
 *  - Return value: one of the BDATTN_* status codes below.
 *
 * Outputs are bfloat16 (the inputs' type); accumulation is float32.
 */
#ifndef BDATTN_H
#define BDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BDATTN_OK = 0,
  BDATTN_ERR_INVALID = 1,      /* null pointer, misaligned pointer, bad size or scale */
  BDATTN_ERR_UNSUPPORTED = 2,  /* head dimension other than 64, 96, 128, 192 or 256 */
  BDATTN_ERR_LAUNCH = 3,       /* the HIP runtime refused a launch */
  BDATTN_ERR_TOO_LARGE = 4,    /* beyond the static scratch of diffusion_attn_bwd_noalloc */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* bdattn_status_string(int status);

/*
 * Forward pass under the block-diffusion mask.
 *   q, k, v : [B][2n][H][D] bf16, tokens 0..n-1 noisy, n..2n-1 clean (read)
 *   out     : [B][2n][H][D] bf16 (written)
 *   lse     : [B][H][2n]   fp32 (written), natural log, includes scale
 * Only key tiles that intersect the mask are read; tiles on a block
 * boundary apply the mask element by element (Fast Diffusion Attention,
 * "Visit only the visible tiles").
 */
int diffusion_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int n, int H, int D, int block_size, float scale, void* stream);

/* Bytes of device workspace diffusion_attn_bwd needs: two float32 values
 * per query row ([B][H][2n] each), -delta_i = -(dout_i . out_i) and the
 * log-sum-exp in base 2.  Returns 0 on bad sizes. */
size_t diffusion_attn_bwd_workspace_size(int B, int n, int H, int D);

/*
 * Backward pass under the block-diffusion mask (FlashAttention: Exact
 * Attention Without Materialization, section 4.5: the probabilities are
 * recomputed from q, k and the saved lse instead of being stored).
 *   q, k, v, out : as produced/consumed by diffusion_attn_fwd (read)
 *   dout         : [B][2n][H][D] bf16, gradient of the loss w.r.t. out (read)
 *   lse          : [B][H][2n] fp32 from diffusion_attn_fwd (read)
 *   dq, dk, dv   : [B][2n][H][D] bf16 (written, fully overwritten)
 *   workspace    : device memory of at least
 *                  diffusion_attn_bwd_workspace_size(B, n, H, D) bytes,
 *                  16-byte aligned; its contents on entry are ignored.
 * dK/dV are produced by a key-major pass over the query tiles that see each
 * key tile, dQ by a separate query-major pass; neither uses atomics, so the
 * result is bitwise reproducible.
 */
int diffusion_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int B, int n, int H, int D, int block_size, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffusion_attn_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the per-row statistics
 * (8 bytes per query row and head) kept in a static device array of the
 * library instead of a caller workspace.  Arguments as diffusion_attn_bwd,
 * without the workspace.
 *   Limit: B * H * 2n <= 4194304 query rows x heads (the array is 32 MiB);
 *   larger problems return BDATTN_ERR_TOO_LARGE and launch nothing.
 *   The array is per GPU: each GPU the library runs on holds its own copy
 *   until the process ends.  The first call on a device looks up its
 *   address there (no allocation); the call runs on the stream's device
 *   (the current device for a NULL stream).
 *   Every call on one GPU uses that GPU's one array, so calls that overlap
 *   in time on the same GPU (other streams, other threads) race and corrupt
 *   each other's results; order them on one stream or with events.  No
 *   state needs clearing between calls: each call writes the statistics of
 *   every row before reading them.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call.
 */
int diffusion_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               int B, int n, int H, int D, int block_size, float scale,
                               void* stream);

/*
 * One stage of the backward pass, for timing the kernels separately.  The
 * arguments are those of the backward entry points below: cu_seqlens NULL
 * for the batched layout (n = half length, or S; total_tokens ignored),
 * non-NULL for packed samples (n = the longest, total_tokens as in the
 * varlen entry points); H_kv = H for plain multi-head attention; mode 0 =
 * diffusion with block_size, 1 = causal (block_size ignored); softcap as
 * in bdattn_fwd (0: off); workspace as bdattn_bwd_workspace_size gives.
 *   stage 0 -- dQ; it also writes the per-row -delta_i = -(dout_i . out_i)
 *              and lse_i * log2(e) to the workspace;
 *   stage 1 -- dK and dV (reads the workspace written by stage 0; with
 *              split groups also the reduction of the partials).
 * The full backward is stages 0 and 1, in that order, on one stream (or
 * with stage 1 ordered after stage 0).  Other stage numbers return
 * BDATTN_ERR_INVALID.
 */
int bdattn_bwd_stage(int mode, int stage, const void* q, const void* k, const void* v,
                     const void* out, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, const int32_t* cu_seqlens, int B, int n, int total_tokens, int H,
                     int H_kv, int D, int block_size, float scale, float softcap,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Causal yardstick forward: q, k, v, out [B][S][H][D] bf16, lse [B][H][S] fp32. */
int causal_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int S, int H, int D, float scale, void* stream);

/* Workspace bytes of causal_attn_bwd (two float32 [B][H][S] arrays). */
size_t causal_attn_bwd_workspace_size(int B, int S, int H, int D);

/* Causal yardstick backward; arguments as diffusion_attn_bwd with T = S. */
int causal_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    int B, int S, int H, int D, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query attention (GQA; multi-query attention when H_kv = 1): the H
 * query heads share H_kv key/value heads.  Query heads form H_kv consecutive
 * groups of H / H_kv; query head h reads key/value head h / (H / H_kv).
 *   q, out, dout, dq : [B][T][H][D]    bf16
 *   k, v, dk, dv     : [B][T][H_kv][D] bf16
 *   lse              : [B][H][T]       fp32 (one per query row, as above)
 * dk and dv of a key/value head are the sums of the gradients that its
 * query heads send it.  The dK/dV kernel walks all query heads of a group
 * for each key tile, so that tile is loaded once for the group and the sum
 * is formed in registers, without atomics (Fast Diffusion Attention,
 * "Ampere and Ada": the GQA-grouped backward).  Requires 1 <= H_kv <= H and
 * H a multiple of H_kv (BDATTN_ERR_INVALID otherwise).  With H_kv = H
 * these compute exactly what the plain entry points compute.
 *
 * When one workgroup per (key tile, sample, key/value head) would leave the
 * GPU short of work (few samples, key/value heads or key tiles), each group
 * is split over several workgroups that write float32 partial dK / dV to
 * the workspace, and a reduction adds the partials in a fixed order: the
 * result is still deterministic.  The *_gqa_workspace_size functions
 * return the bytes this needs: the per-row statistics of the plain entry
 * points, plus the partials when the groups are split: about
 * 2 * W * K * D * 4 bytes for a split grid of W dK/dV workgroups of K
 * keys each (K = 128, or 64 at D = 256), where
 * groups are split only while the unsplit grid is under 1024 workgroups
 * (2048 at D = 64 and 96), so W stays below 4096 when H / H_kv is a power
 * of two.
 * They return 0 on bad sizes.
 */
size_t diffusion_attn_bwd_gqa_workspace_size(int B, int n, int H, int H_kv, int D);
size_t causal_attn_bwd_gqa_workspace_size(int B, int S, int H, int H_kv, int D);
int diffusion_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* stream);
int diffusion_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);
int causal_attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int S, int H, int H_kv, int D, float scale, void* stream);
int causal_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int S, int H, int H_kv, int D, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward pass (Fast Diffusion Attention, "Results": the FP8 forward).
 *   q                : [B][T][H][D]    OCP FP8 E4M3 bytes (1 sign, 4 exponent
 *                      bits with bias 7, 3 mantissa bits; largest value 448)
 *   k, v             : [B][T][H_kv][D] E4M3 bytes
 *   q_descale        : [B][H] float32, k_descale and v_descale [B][H_kv]:
 *                      the value a byte stands for is descale * e4m3(byte)
 *   out              : [B][T][H][D] bf16;  lse : [B][H][T] fp32 (natural log)
 * The scores are scale * q_descale * k_descale * (q . k) with the products
 * of the E4M3 values accumulated in float32.  The softmax runs in float32;
 * its unnormalised probabilities 2^(s log2(e) - m) (m within 8 of the row
 * maximum, so at most 2^8) are rounded to E4M3 for the P.V product, and
 * the denominator sums the unrounded values.  That rounding is the one
 * approximation beyond the bf16 pass: it moves an output element by at
 * most 2^-4 sum_j P_ij |v_j| + 2^-10 sum_j |v_j| / l_i (l_i the row sum at
 * the maximum).  T = 2n (diffusion, block_size as above) or S (causal).
 * Grouped heads as in the _gqa entry points.  Same pointer, size and
 * error rules as diffusion_attn_fwd, plus: the descale arrays must be
 * non-NULL and 4-byte aligned, and D must be 64 or 128
 * (BDATTN_ERR_UNSUPPORTED for 96, 192 and 256).  There is no FP8 backward.
 */
int diffusion_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                           const float* k_descale, const float* v_descale, void* out, float* lse,
                           int B, int n, int H, int H_kv, int D, int block_size, float scale,
                           void* stream);
int causal_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, const float* v_descale, void* out, float* lse,
                        int B, int S, int H, int H_kv, int D, float scale, void* stream);

/*
 * Packed batches of samples of different lengths (Fast Diffusion
 * Attention, "Hopper": varlen batches, as in supervised fine-tuning).
 *   cu_seqlens : B + 1 int32 token offsets in device memory, 4-byte aligned
 *                (read by the kernels, never by the host): sample b holds
 *                the packed tokens [cu_seqlens[b], cu_seqlens[b+1]), laid
 *                out [noisy n_b | clean n_b] (diffusion, 2 n_b tokens) or
 *                as one sequence of S_b tokens (causal).  Samples may be
 *                empty.
 *   max_n      : the largest n_b (max_S: the largest S_b), >= 1; it sizes
 *                the grid, whose workgroups past a sample's end exit at
 *                once, heaviest tiles first.
 *   total_tokens : packed tokens (rows of q); 0 computes nothing and
 *                returns BDATTN_OK.
 *   q, out, dout, dq : [total_tokens][H][D] bf16
 *   k, v, dk, dv     : [total_tokens][H_kv][D] bf16 (grouped heads as above)
 *   lse              : [H][total_tokens] fp32
 * Each sample is computed exactly as the batched entry points compute it
 * on that sample alone.  A sample whose offsets are inconsistent
 * (negative, decreasing, past total_tokens, an odd diffusion length, or
 * longer than max_n) is skipped and its outputs are undefined; nothing
 * outside the tensors is accessed.  Rows outside every sample are not
 * written.  The workspace sizes follow the rules of the grouped backward,
 * with total_tokens rows.
 */
int diffusion_attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              const int32_t* cu_seqlens, int B, int max_n, int total_tokens,
                              int H, int H_kv, int D, int block_size, float scale, void* stream);
size_t diffusion_attn_varlen_bwd_workspace_size(int B, int max_n, int total_tokens, int H,
                                                int H_kv, int D);
int diffusion_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens, int B, int max_n, int total_tokens,
                              int H, int H_kv, int D, int block_size, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);
int causal_attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* cu_seqlens, int B, int max_S, int total_tokens, int H,
                           int H_kv, int D, float scale, void* stream);
size_t causal_attn_varlen_bwd_workspace_size(int B, int max_S, int total_tokens, int H, int H_kv,
                                             int D);
int causal_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           const int32_t* cu_seqlens, int B, int max_S, int total_tokens, int H,
                           int H_kv, int D, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * The general form of the bf16 passes: every option in one call.
 *   mode        : 0 = block diffusion (T = 2n, block_size), 1 = causal (T = n)
 *   cu_seqlens  : NULL for the batched layout [B][T][heads][D] (n = half or
 *                 sequence length, total_tokens ignored); non-NULL for
 *                 packed samples as in the varlen entry points (n = the
 *                 longest; total_tokens = 0 computes nothing)
 *   H, H_kv     : query and key/value heads (grouped as in the _gqa entry
 *                 points; H_kv = H for plain multi-head attention)
 *   softcap     : 0 = off; > 0 caps the scaled scores s to
 *                 softcap * tanh(s / softcap) before the softmax (the
 *                 softcapping Fast Diffusion Attention lists among what its
 *                 tests cover, "Accuracy"; defined as in flash-attention),
 *                 and the backward takes the cap's derivative into dS.
 *                 Must be finite and >= 0.
 * Tensors, workspace and errors as in the specific entry points, which are
 * this call with softcap = 0.  bdattn_bwd_workspace_size takes packed = 0
 * or 1 for the two layouts (the workspace does not depend on softcap).
 */
int bdattn_fwd(int mode, const void* q, const void* k, const void* v, void* out, float* lse,
               const int32_t* cu_seqlens, int B, int n, int total_tokens, int H, int H_kv, int D,
               int block_size, float scale, float softcap, void* stream);
size_t bdattn_bwd_workspace_size(int mode, int packed, int B, int n, int total_tokens, int H,
                                 int H_kv, int D);
int bdattn_bwd(int mode, const void* q, const void* k, const void* v, const void* out,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               const int32_t* cu_seqlens, int B, int n, int total_tokens, int H, int H_kv, int D,
               int block_size, float scale, float softcap, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * Host-side inspection of the tile enumeration the kernels use (pure integer
 * logic, no GPU needed).  Fast Diffusion Attention, "Visit only the visible
 * tiles": the halves are tiled independently (no tile covers tokens of both
 * halves).  Clean query rows only ever need clean key tiles from the start
 * of the half through their own block; noisy query rows need the clean key
 * tiles that precede their blocks plus the noisy key tiles that overlap
 * their own blocks.  Nothing else is visited.
 *
 * mode: 0 = diffusion (halves 0 = noisy, 1 = clean), 1 = causal (one
 * sequence of length n, reported as half 1).  Tiles are tile_m query rows by
 * tile_n keys, aligned to multiples of their size inside each half.
 *
 * bdattn_fwd_tiles lists, for query tile qt of half qhalf, every visited key
 * tile as 3 int32 entries {key_half, key_tile, masked}; masked = 1 when the
 * tile needs the element mask (some pair inside it is invisible), 0 when
 * every pair is visible.  bdattn_bwd_tiles lists, for key tile kt of half
 * khalf, every query tile that sees it as {query_half, query_tile, masked}.
 * Both write at most max_entries entries and return the number of visited
 * tiles (which may exceed max_entries), or -1 on bad arguments.
 */
int bdattn_fwd_tiles(int mode, int n, int block_size, int tile_m, int tile_n,
                     int qhalf, int qt, int32_t* entries, int max_entries);
int bdattn_bwd_tiles(int mode, int n, int block_size, int tile_m, int tile_n,
                     int khalf, int kt, int32_t* entries, int max_entries);

/* Visible key interval [lo, hi) of query row p of half qhalf within key half
 * khalf (positions inside that half); lo == hi when it sees none of it.
 * Returns 0, or -1 on bad arguments. */
int bdattn_row_interval(int mode, int n, int block_size, int qhalf, int p, int khalf,
                        int32_t* lo, int32_t* hi);

/* Visible (query, key) pairs of one (sample, head): the sum over rows of
 * their visible interval lengths.  -1 on bad arguments. */
int64_t bdattn_visible_pairs(int mode, int n, int block_size);

#ifdef __cplusplus
}
#endif

#endif /* BDATTN_H */
