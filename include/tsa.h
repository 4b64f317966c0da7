/*
 * tsa.h -- C ABI of the token-pruned self-attention library (libtsa.so, gfx950).
 *
 * One pruned attention layer step over video-DiT latent tokens:
 *   score -> select -> compact -> QKV of the active tokens -> KV-cache sync
 *   -> attention of the active queries over the whole cache -> scatter.
 *
 * Step labels used in the comments below:
 *   a1 score, a2 select, a3 compact, a4 gather (optionally with recovery),
 *   a5 QKV projection, a6 KV-cache sync, a7 attention, a8 scatter;
 *   f1 cached Euler update, f2 long/short-term pruning mask and frame
 *   restoration, f3 3D rotary positions and frame-causal attention,
 *   f4 Timeripple partial-score reuse (the steps beside the layer).
 *
 * Sources, cited by page title and section (gist.science summaries):
 *   [HSA]   "Resumen Técnico: Asignación de Pasos Heterogénea (HSA) para la
 *           Generación Eficiente de Video", gist.science/es/paper/2605.06892
 *   [LIPAR] "Training-free Latent Inter-Frame Pruning with Attention Recovery",
 *           gist.science/es/paper/2603.05811 (and the Dutch page /nl/)
 *   [Timeripple] "Resumen Técnico: TIMERIPPLE", gist.science/es/paper/2511.12035
 *
 * Conventions shared by every call
 *   - Pointers named *device* are device (HBM) addresses owned by the caller;
 *     the library never allocates, frees or keeps them.  Pointers named *host*
 *     are read during the call only.
 *   - Token rows are row-major [rows, dim]; inside Q/K/V, column h*head_dim+j
 *     is dimension j of head h.  bf16 values are passed as raw 16-bit words
 *     (tsa_bf16).  Row buffers must be 16-byte aligned.
 *   - Index lists are int32, ascending, without repeats, within range.  This
 *     is a precondition: the release build's kernels clamp nothing and do not
 *     check it.  The debug build (libtsa_debug.so, compiled with TSA_DEBUG)
 *     checks every index list on the GPU before a kernel reads it and returns
 *     TSA_ERR_SHAPE for a violation (synchronising the stream to do so);
 *     query-token lists are only checked to be non-negative.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises.  Device faults
 *     surface at the caller's next synchronisation.
 *   - A call with n == 0 rows of work returns TSA_OK and enqueues nothing.
 *   - Arguments are validated before anything is enqueued; a failed
 *     validation returns an error code and writes nothing.
 */
#ifndef TSA_H
#define TSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSA_ABI_VERSION 7

typedef uint16_t tsa_bf16;

typedef enum tsa_status {
  TSA_OK = 0,
  TSA_ERR_INVALID_ARG = 1, /* NULL where a buffer is required, unknown enum value */
  TSA_ERR_SHAPE = 2,       /* sizes out of range or inconsistent */
  TSA_ERR_DTYPE = 3,       /* element type not supported by this call */
  TSA_ERR_ALIGNMENT = 4,   /* a row buffer is not 16-byte aligned */
  TSA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  TSA_ERR_HIP = 6          /* the HIP runtime refused a launch */
} tsa_status;

typedef enum tsa_dtype { TSA_F32 = 0, TSA_BF16 = 1 } tsa_dtype;

typedef enum tsa_score_kind {
  TSA_SCORE_REL_L1 = 0, /* sum|x - r| / sum|r|   ([HSA] §2.1, dynamic token selection) */
  TSA_SCORE_ABS_L1 = 1  /* sum|x - r|            ([LIPAR] §2.B, L1 change vs threshold) */
} tsa_score_kind;

typedef enum tsa_select_mode {
  TSA_SELECT_TOPK = 0,      /* the k highest scores; equal scores taken in ascending token order */
  TSA_SELECT_THRESHOLD = 1, /* active iff score >= tau; below tau is redundant ([LIPAR] §2.B) */
  TSA_SELECT_MASK = 2,      /* active iff aux_in[n] != 0 (a caller-given set) */
  TSA_SELECT_SCHEDULE = 3   /* active iff step mod aux_in[n] == 0, aux_in = period T/s_k ([HSA] §2.1) */
} tsa_select_mode;

/* Version of this ABI (TSA_ABI_VERSION of the build). */
int tsa_abi_version(void);

/* Static text for a status code ("unknown status" for other values). */
const char* tsa_status_string(int status);

/* Bytes of device workspace tsa_select_active / tsa_assign_groups need for n_rows tokens (may be 0). */
size_t tsa_select_workspace_bytes(int64_t n_rows);

/*
 * a1-a3: score every token, select the active set A_i, compact it.
 * [HSA] §2.1 (relative L1 change per token ranks tokens), [LIPAR] §2.B
 * (L1 change of a latent patch against the same location in the previous
 * frame; below the threshold the patch is pruned), [HSA] §2.2 item 1 (only
 * the active subset goes on).
 *
 *   x_cur        device, [n_rows, dim] of `dtype` (TSA_F32 or TSA_BF16).
 *   x_ref        device, [n_rows, dim] of `dtype`, or NULL to use x_cur itself.
 *   ref_row_offset  the reference row of token n is ref[n - ref_row_offset];
 *                tokens with no such row (n - offset outside [0, n_rows)) score
 *                +inf, so top-k and threshold keep them.  0 = same row of x_ref;
 *                H*W with x_ref = NULL = same location one frame earlier.
 *   score_kind   tsa_score_kind.  Relative: 0/0 scores 0, x/0 scores +inf.
 *   mode         tsa_select_mode.  TOPK uses k (0 <= k <= n_rows), THRESHOLD
 *                uses tau, MASK and SCHEDULE read aux_in (device u8[n_rows])
 *                and do not compute scores; SCHEDULE also uses `step` (>= 0),
 *                and a period of 0 means never active.
 *   scores_out   device f32[n_rows]; required for TOPK and THRESHOLD, unused
 *                (may be NULL) for MASK and SCHEDULE.
 *   mask_out     device u8[n_rows] (1 = active), required.
 *   idx_out      device i32[n_rows] capacity, required: entries [0, n_active)
 *                are the active tokens in ascending order.
 *   pidx_out     device i32[n_rows] capacity or NULL: entries
 *                [0, n_rows - n_active) are the pruned tokens, ascending.
 *   n_active_out device i32[1], required.
 *   workspace    device, tsa_select_workspace_bytes(n_rows) bytes (NULL if 0).
 * Errors: INVALID_ARG, SHAPE (n_rows < 0 or >= 2^31, dim <= 0 or dim % 8,
 * k out of range, step < 0), DTYPE, ALIGNMENT, WORKSPACE, HIP.
 */
tsa_status tsa_select_active(const void* x_cur, const void* x_ref, int64_t ref_row_offset,
                             int64_t n_rows, int64_t dim, int dtype, int score_kind, int mode,
                             int64_t k, float tau, const uint8_t* aux_in, int64_t step,
                             float* scores_out, uint8_t* mask_out, int32_t* idx_out,
                             int32_t* pidx_out, int32_t* n_active_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * a1 alone (for measurement and for callers that select on the host): the
 * per-token change scores of tsa_select_active, with the same reference-row
 * rules and the same arithmetic, written to scores_out (device f32[n_rows]).
 * Errors: INVALID_ARG, SHAPE, DTYPE, ALIGNMENT, HIP.
 */
tsa_status tsa_token_scores(const void* x_cur, const void* x_ref, int64_t ref_row_offset, int64_t n_rows,
                            int64_t dim, int dtype, int score_kind, float* scores_out, void* stream);

/*
 * [HSA] §2.1: partition the tokens into disjoint groups by score rank
 * (highest score first, ties in ascending token order): group g takes the
 * next group_counts[g] tokens and each of its tokens gets the activity period
 * group_periods[g] (= T / s_g).  The result feeds TSA_SELECT_SCHEDULE.
 *
 *   scores         device f32[n] (e.g. scores_out of tsa_select_active).
 *   n_groups       1..16.
 *   group_counts   host int64[n_groups], each >= 0, summing to n.
 *   group_periods  host uint8[n_groups].
 *   period_out     device u8[n].
 *   workspace      device, tsa_select_workspace_bytes(n) + n bytes.
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
tsa_status tsa_assign_groups(const float* scores, int64_t n, int n_groups,
                             const int64_t* group_counts, const uint8_t* group_periods,
                             uint8_t* period_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * a4-a5 (+ optional a6): project token rows through the fused QKV weight.
 * [HSA] §2.2 item 1: only the active tokens go through the Q/K/V projections.
 * [LIPAR] §2.C (noise-aware duplication): a pruned token's K/V come from its
 * clean previous latent re-noised with fresh noise.
 *
 * Row r of the product takes its input from token t = rows[r] (or t = r when
 * rows is NULL):
 *   eps == NULL:  A[r] = x[t]                         (x of `x_dtype`, converted to bf16)
 *   eps != NULL:  A[r] = bf16((1 - sigma) * x[t - src_row_offset] + sigma * eps[t])
 *                 computed in fp32 and rounded to nearest even; a token whose
 *                 row t - src_row_offset is outside [0, n_x_rows) takes 0 for
 *                 the first term.  x must then be TSA_BF16.
 * and Q/K/V[r] = bf16(A[r] @ W_part^T), fp32 accumulation, nearest-even rounding.
 *
 *   x            device [n_x_rows, dim] of x_dtype (TSA_F32 or TSA_BF16).
 *   rows         device i32[n] token indices into x (each in [0, n_x_rows)), or NULL.
 *   w_qkv        device bf16 [3*dim, dim]; rows [0,dim) = W_q, [dim,2dim) = W_k,
 *                [2dim,3dim) = W_v (output feature-major, like a linear layer).
 *   q_out        device bf16 [n, dim] (compact row r), or NULL to skip Q.
 *   k_out/v_out  device bf16, required.  out_is_cache == 0: compact [n, dim].
 *                out_is_cache != 0: the caches [n_cache, dim]; row r is written
 *                to row rows[r] (rows required, each < n_cache) -- this fuses
 *                the cache sync (a6) into the projection.
 *   eps          device bf16 [n_x_rows, dim] or NULL (no recovery).
 * dim must be a multiple of 64; 3*dim*dim*2 must be below 2^31 bytes (the weight
 * is one 32-bit buffer range).  x of any size (token rows of 2^31 bytes or more
 * are read through 64-bit addresses).
 * Errors: INVALID_ARG, SHAPE, DTYPE, ALIGNMENT, HIP.
 */
tsa_status tsa_qkv_active(const void* x, int x_dtype, int64_t n_x_rows, const int32_t* rows,
                          int64_t n, int64_t dim, const tsa_bf16* w_qkv, tsa_bf16* q_out,
                          tsa_bf16* k_out, tsa_bf16* v_out, int out_is_cache, int64_t n_cache,
                          const tsa_bf16* eps, int64_t src_row_offset, float sigma,
                          void* stream);

/*
 * tsa_qkv_active with 3D rotary positions on Q and K (the RoPE of video DiTs:
 * [Timeripple] Metodología §1 describes its channels split into a temporal
 * group and two spatial groups; [LIPAR] §2.C).  Token t sits at frame
 * t / (height*width), row (t / width) % height, column t % width.  Each
 * head's head_dim = dim / heads channels are split into time / height / width
 * groups of head_dim - 4*(head_dim/6), 2*(head_dim/6), 2*(head_dim/6)
 * channels; inside the group of an axis of size n, channel pair (2i, 2i+1)
 * is rotated by the angle pos * rope_base^(-2i/n) (pos = the token's
 * coordinate on that axis), in fp32 on the fp32 product, before the single
 * bf16 rounding.  V is not rotated; the cache therefore holds rotated K.
 * Arguments as tsa_qkv_active, plus heads (head_dim even, >= 6), height,
 * width >= 1 and rope_base > 0 (finite).
 * Errors: INVALID_ARG, SHAPE, DTYPE, ALIGNMENT, HIP.
 */
tsa_status tsa_qkv_active_rope(const void* x, int x_dtype, int64_t n_x_rows, const int32_t* rows,
                               int64_t n, int64_t dim, const tsa_bf16* w_qkv, tsa_bf16* q_out,
                               tsa_bf16* k_out, tsa_bf16* v_out, int out_is_cache, int64_t n_cache,
                               const tsa_bf16* eps, int64_t src_row_offset, float sigma, int heads,
                               int64_t height, int64_t width, float rope_base, void* stream);

/*
 * a4-a6 for rows prepared beforehand: [LIPAR] §2.C recovered rows gathered once
 * into a compact buffer (tsa_gather_rows) and projected here, so the recovery
 * arithmetic runs once per row instead of once per output-feature tile.
 * Row r of the product reads a[r] and belongs to token t = rows[r]:
 *   K/V[r] = bf16(a[r] @ W_k/v^T) written to cache row t; Q[r] likewise to
 * q_out[r] (compact) when q_out is not NULL.  heads > 0: Q and K rotated by the
 * 3D position of token t as in tsa_qkv_active_rope ([Timeripple] Metodología §1).
 *   a          device bf16 [n, dim].
 *   rows       device i32[n], each < n_cache.
 *   w_qkv      as in tsa_qkv_active.
 *   k_cache, v_cache  device bf16 [n_cache, dim].
 *   heads, height, width, rope_base  rotary positions (heads = 0: none).
 * dim a multiple of 64; 3*dim*dim*2 below 2^31 bytes; a of any size.
 * Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
tsa_status tsa_qkv_rows_to_cache(const tsa_bf16* a, int64_t n, int64_t dim, const int32_t* rows,
                                 const tsa_bf16* w_qkv, tsa_bf16* q_out, tsa_bf16* k_cache, tsa_bf16* v_cache,
                                 int64_t n_cache, int heads, int64_t height, int64_t width, float rope_base,
                                 void* stream);

/*
 * a6: [HSA] §2.2 item 2 -- the fresh K/V of the active tokens overwrite
 * their rows of the per-layer cache; every other row keeps its stale entry.
 *   k_a, v_a          device bf16 [n, dim] (compact, row r belongs to token rows[r]).
 *   rows              device i32[n], each in [0, n_cache).
 *   k_cache, v_cache  device bf16 [n_cache, dim], updated in place.
 * dim must be a multiple of 8.  Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
tsa_status tsa_kv_cache_sync(const tsa_bf16* k_a, const tsa_bf16* v_a, const int32_t* rows,
                             int64_t n, tsa_bf16* k_cache, tsa_bf16* v_cache, int64_t n_cache,
                             int64_t dim, void* stream);

/*
 * a7: [HSA] §2.2 items 3-4 -- the active queries attend over the full cached
 * K/V (fresh rows for active tokens, stale rows for skipped ones); cost
 * O(|A_i| * N) instead of O(N^2).  Per head h:
 *   O[r, h] = softmax_j(scale * Q[r, h] . K[j, h]) V[j, h],  j over all n_kv rows,
 * no mask (bidirectional).  bf16 inputs, fp32 accumulation and softmax,
 * bf16 output (nearest even).
 *
 *   q        device bf16 [n_q, heads*head_dim].
 *   k_cache, v_cache  device bf16 [n_kv, heads*head_dim], n_kv >= 1.
 *   head_dim 64 or 128; heads >= 1.
 *   scale    > 0, or <= 0 for 1/sqrt(head_dim).
 *   out      device bf16: out_rows == NULL: compact [n_q, dim];
 *            otherwise [n_out, dim] with row r written to row out_rows[r]
 *            (this fuses the scatter, a8); other rows are not touched.
 *   lse_out  device f32 [heads, n_q] natural-log normaliser log sum_j exp(scale*s_j), or NULL.
 *   workspace  device memory of at least tsa_attention_workspace_bytes() bytes for
 *            the same n_q, n_kv, heads, head_dim on the current device, or NULL.
 *            The query tiles (256 queries of one head for head_dim 128, 128 for
 *            64) run one per workgroup.  With a workspace, when the last round
 *            of tiles would leave compute units idle, each tile of that round
 *            is instead cut into key ranges run by workgroups of their own; they
 *            leave fp32 partials in the workspace and a second small kernel on
 *            the same stream combines them.  NULL: no split.  Results agree to
 *            rounding; the workspace keeps nothing between calls, and calls that
 *            run concurrently need separate workspaces.
 * Any cache size up to n_kv < 2^31 rows: caches of 2^31 bytes or more run kernels
 * that rebase their 32-bit buffer ranges at every key tile.
 * Errors: INVALID_ARG, SHAPE, ALIGNMENT, WORKSPACE (workspace non-NULL and
 * workspace_bytes below the required size), HIP.
 */
tsa_status tsa_sparse_query_attention(const tsa_bf16* q, const tsa_bf16* k_cache,
                                      const tsa_bf16* v_cache, int64_t n_q, int64_t n_kv,
                                      int heads, int head_dim, float scale, tsa_bf16* out,
                                      const int32_t* out_rows, int64_t n_out, float* lse_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Frame-causal variant of tsa_sparse_query_attention (causal video models:
 * [LIPAR] §3-§4, causal Self-Forcing as well as bidirectional models): the
 * query of token t = q_tokens[r] attends only to the keys of the frames up to
 * its own, j < (t / frame_tokens + 1) * frame_tokens (capped at n_kv); a
 * block-causal mask with one block per frame of frame_tokens tokens.  Every
 * query sees at least key 0.  Same arguments, layouts and rounding as
 * tsa_sparse_query_attention otherwise (no split schedule).
 *   q_tokens     device i32[n_q], token index of each query row, >= 0.
 *   frame_tokens tokens per frame (H*W), >= 1.
 * Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
tsa_status tsa_frame_causal_attention(const tsa_bf16* q, const tsa_bf16* k_cache, const tsa_bf16* v_cache,
                                      int64_t n_q, int64_t n_kv, int heads, int head_dim, float scale,
                                      const int32_t* q_tokens, int64_t frame_tokens, tsa_bf16* out,
                                      const int32_t* out_rows, int64_t n_out, float* lse_out, void* stream);

/*
 * Workspace size for tsa_sparse_query_attention on the current device (the
 * split depends on its compute-unit count); 0 when no split pays off or the
 * shape is invalid.  Never more than 6 partials of 256 x 128 (head_dim 128) or
 * 128 x 64 (head_dim 64) fp32 values plus 2 per query per resident workgroup:
 * 207 MB for head_dim 128 on a 256-CU GPU.
 */
size_t tsa_attention_workspace_bytes(int64_t n_q, int64_t n_kv, int heads, int head_dim);

/*
 * a8: outputs of the active tokens go back to token order; rows not listed
 * keep their previous value ([HSA] §2.3: skipped tokens reuse what was cached).
 *   o_a   device bf16 [n, dim];  rows device i32[n] in [0, n_out);  out device bf16 [n_out, dim].
 * dim must be a multiple of 8.  Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
tsa_status tsa_scatter_out(const tsa_bf16* o_a, const int32_t* rows, int64_t n, tsa_bf16* out,
                           int64_t n_out, int64_t dim, void* stream);

/*
 * a4 alone (for measurement and for callers that keep a compact copy):
 * dst[r] = bf16 row source of token rows[r], with the same row-source rules
 * as tsa_qkv_active (plain gather, or recovery when eps != NULL).
 *   x    device bf16 [n_x_rows, dim];  rows device i32[n];  dst device bf16 [n, dim].
 * dim must be a multiple of 8.  Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
tsa_status tsa_gather_rows(const tsa_bf16* x, int64_t n_x_rows, const int32_t* rows, int64_t n,
                           int64_t dim, const tsa_bf16* eps, int64_t src_row_offset, float sigma,
                           tsa_bf16* dst, void* stream);

/*
 * [HSA] §2.3 cached Euler update: after a global step every token, active or
 * skipped, advances by the same increment dt = sigma_{i+1} - sigma_i along
 * its cached velocity (the velocity of its most recent active step):
 *   x[r, j] <- x[r, j] + dt * v_hat[r, j]   for all n_rows rows,
 * computed as one fused multiply-add in fp32 (TSA_F32 state: rounded once;
 * TSA_BF16 state: that result rounded to nearest even).
 *   x       device [n_rows, dim] of x_dtype, updated in place.
 *   v_hat   device bf16 [n_rows, dim] (e.g. the layer output in token order,
 *           whose skipped rows keep their last active value).
 * dim must be a multiple of 8; dt finite.  Errors: INVALID_ARG, SHAPE, DTYPE,
 * ALIGNMENT, HIP.
 */
tsa_status tsa_euler_update(void* x, int x_dtype, const tsa_bf16* v_hat, int64_t n_rows, int64_t dim,
                            float dt, void* stream);

/*
 * [LIPAR] §2.B pruning mask with short- and long-term changes.  Tokens are
 * frame-major, token t = f * hw + l for frame f and spatial location l.  For
 * f >= 1 the short-term change compares row t with the same location in
 * frame f-1, the long-term change with the same location in the most recent
 * earlier frame where that location was kept; changes are L1 norms of the
 * row difference (TSA_SCORE_REL_L1: divided by the L1 norm of the reference
 * row, 0/0 -> 0, x/0 -> +inf).  Token t is pruned (mask 0) iff
 * short < tau_short and long < tau_long; frame 0 is always kept (mask 1,
 * scores +inf).  Sums in fp32, fixed order.
 *   x          device [frames * hw, dim] of dtype (TSA_F32 or TSA_BF16).
 *   mask_out   device u8[frames * hw].
 *   short_out, long_out  device f32[frames * hw] or NULL.
 * dim must be a multiple of 8, at most 8192 (bf16) or 4096 (fp32); the
 * thresholds must not be NaN (+inf allowed).  The mask feeds
 * tsa_select_active in TSA_SELECT_MASK mode.
 * Errors: INVALID_ARG, SHAPE, DTYPE, ALIGNMENT, HIP.
 */
tsa_status tsa_lif_mask(const void* x, int dtype, int64_t frames, int64_t hw, int64_t dim, int score_kind,
                        float tau_short, float tau_long, uint8_t* mask_out, float* short_out,
                        float* long_out, void* stream);

/*
 * [LIPAR] (Dutch page) §2.D restoration: after denoising, every pruned token
 * (mask 0) is filled in with the same location of the previous frame, so the
 * result is a full token sequence; along the frame axis this carries the most
 * recent kept row forward.  Kept rows and frame-0 rows are not written.
 *   buf    device [frames * hw, dim] of dtype, frame-major as in tsa_lif_mask,
 *          updated in place.
 *   mask   device u8[frames * hw].
 * dim must be a multiple of 8.  Errors: INVALID_ARG, SHAPE, DTYPE, ALIGNMENT, HIP.
 */
tsa_status tsa_restore_frames(void* buf, int dtype, const uint8_t* mask, int64_t frames, int64_t hw,
                              int64_t dim, void* stream);

/* Bytes of device workspace tsa_timeripple_reuse needs: 2 * n_rows * heads * 3 * 4. */
size_t tsa_reuse_workspace_bytes(int64_t n_rows, int heads);

/*
 * [Timeripple] Metodología §1-§2: partial attention scores of Q or K tokens
 * reused from neighbouring tokens.  A head's channels form the rotary groups
 * time [0, d_t), height [d_t, d_t + d_s), width [d_t + d_s, d) with
 * d_s = 2 * (d / 6), d_t = d - 2 * d_s.  For token t (frame-major: frame
 * t / (height*width), row (t / width) % height, column t % width), head h and
 * axis a (0 time, 1 height, 2 width), with nb_a(t) the token one frame, row or
 * column back:
 *   delta[t,h,a] = ||v[t,h,C_a] - v[nb_a(t),h,C_a]||_2 / ||v[t,h,C_a]||_2
 * over C_a = the channels of the two groups axis a does not rotate (0/0 -> 0,
 * x/0 -> +inf; +inf when there is no neighbour), sums in fp32.  Group g of
 * token t takes its channels from the neighbour along the first axis a != g
 * (order time, height, width) with delta[t,h,a] < thetas[a]; from itself when
 * there is none.  Sources are followed back to the token that keeps the group's
 * own channels, so
 *   v_eff[t, h, group g] = v[root(t, h, g), h, group g],
 * and attention of (Q_eff, K_eff, V) is attention with reused partial scores.
 *   v          device bf16 [n_rows, heads * head_dim] (Q or K, rotary positions
 *              already applied); must not overlap v_eff.
 *   thetas     host float[3] (time, height, width), each >= 0 or +inf, not NaN.
 *   v_eff      device bf16 [n_rows, heads * head_dim].
 *   src_out    device i32[n_rows, heads, 3] (the immediate source token of each
 *              group) or NULL.
 *   delta_out  device f32[n_rows, heads, 3] (delta per axis) or NULL.
 *   workspace  device, at least tsa_reuse_workspace_bytes(n_rows, heads) bytes,
 *              4-byte aligned.
 * head_dim 64 or 128; height, width >= 1.
 * Errors: INVALID_ARG, SHAPE, ALIGNMENT, WORKSPACE, HIP.
 */
tsa_status tsa_timeripple_reuse(const tsa_bf16* v, int64_t n_rows, int heads, int head_dim, int64_t height,
                                int64_t width, const float* thetas, tsa_bf16* v_eff, int32_t* src_out,
                                float* delta_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tsa_timeripple_reuse without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The source and root tables live in a static device
 * array of the library (24 MiB on each GPU it runs on, held until the process
 * ends), so n_rows * heads may be at most tsa_reuse_noalloc_max_token_heads()
 * (2^20).  Every call on one GPU uses that GPU's single array: calls that overlap
 * on one GPU (several streams or host threads) race and must be ordered by the
 * caller.  Nothing is allocated and no allocating routine is called.  Arguments,
 * results and errors as tsa_timeripple_reuse; SHAPE also when n_rows * heads is
 * above the maximum.
 */
tsa_status tsa_timeripple_reuse_noalloc(const tsa_bf16* v, int64_t n_rows, int heads, int head_dim, int64_t height,
                                        int64_t width, const float* thetas, tsa_bf16* v_eff, int32_t* src_out,
                                        float* delta_out, void* stream);

/* Largest n_rows * heads tsa_timeripple_reuse_noalloc accepts (2^20). */
size_t tsa_reuse_noalloc_max_token_heads(void);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H */
