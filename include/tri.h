/*
 * tri.h - C interface of libtri: the key-eviction pass of TriAttention on MI355X (gfx950).
 *
 * One pass over a KV cache made of independent *units* (one KV head of one layer of one
 * sequence) does three things:
 *   1. scores every cached key with the offset-averaged trigonometric score, folded into
 *      one complex weight per rotary band;
 *   2. keeps the B highest-scoring keys of each unit;
 *   3. copies the kept K/V rows and positions into dense per-unit buffers.
 *
 * Sources (cited by title and section):
 *   [N] "The future-offset average in TriAttention can be precomputed" (A. Mukherjee):
 *       "The score TriAttention computes", "The same score, read as arrows in the plane",
 *       "The averaging step", "What it saves, and what it does not".
 *   [R] TriAttention project README: KV budget settings for serving and chat.
 *
 * Notation: d = head dimension (even), F = d/2 rotary bands, U = units, N_u = cached keys of
 * unit u, B = budget (rows kept per unit), t_u = current position of unit u, p = a key's
 * position, delta = t_u - p. Band f of a d-vector x is the complex number x[2f] + i*x[2f+1]
 * ("interleaved" pairs). omega_f = theta^(-2f/d) ([N] "The score TriAttention computes").
 *
 * Conventions shared by every entry point:
 *  - Return value: TRI_OK (0) or a negative TRI_ERR_* code. Nothing throws across the ABI.
 *  - All argument checks run on the host before any HIP call; when a check fails nothing is
 *    enqueued and no output is touched.
 *  - The caller owns every buffer. The library allocates no device memory and keeps no state
 *    between calls, except what a caller-provided workspace holds between the calls of one
 *    pass (the histogram from tri_score to tri_select_topb), and the static workspace array of
 *    tri_prune_pass_noalloc.
 *  - Device entry points are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream). Nothing synchronises the host.
 *  - Device pointers must be 16-byte aligned unless stated otherwise.
 *  - Device-side preconditions that the host cannot check (row_off contents, positions) are
 *    stated per function. Kernels clamp every row range to [0, total_rows), so a broken
 *    row_off yields wrong values, never an access outside the buffers.
 */
#ifndef TRI_H
#define TRI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TRI_OK               0
#define TRI_ERR_ARG         -1  /* bad size, pointer, alignment or enum value */
#define TRI_ERR_UNSUPPORTED -2  /* valid request that the library does not implement */
#define TRI_ERR_ALIAS       -3  /* an output range overlaps an input range or another output */
#define TRI_ERR_WORKSPACE   -4  /* workspace missing or smaller than required */
#define TRI_ERR_HIP         -5  /* the HIP runtime reported an error at launch */

/* element types of K and V */
#define TRI_DT_F32  0  /* IEEE binary32 */
#define TRI_DT_BF16 1  /* bfloat16 (upper half of a binary32) */

/* how the d coordinates of a key pair up into F complex bands */
#define TRI_BANDS_INTERLEAVED 0  /* band f = (x[2f], x[2f+1]) */
#define TRI_BANDS_HALF_SPLIT  1  /* band f = (x[f], x[f + d/2]) (rotate-half storage) */
/* OR-ed into a layout: the keys are stored after the rotary rotation at their own positions,
 * band f holding k_f * e^{i omega_f pos} (see tri_score) */
#define TRI_KEYS_ROTATED 0x100

/* flags of tri_select_topb */
#define TRI_SELECT_HIST_FROM_SCORE 1u  /* ws holds the histogram tri_score accumulated */

/* Short English text for a status code (static storage; never NULL). */
const char* tri_status_string(int status);

/*
 * tri_fold_weights - offline fold of the offset schedule into one weight per band.
 *
 *   W_f    = (1/|D|) * sum_{delta in D} e^{i omega_f delta}                 (f = 0 .. F-1)
 *   mu'_f  = E[q_f] * W_f                        per unit, the offset-averaged center
 *
 * [N] "The averaging step": the average over future offsets touches only the rotation
 * factor e^{i omega_f delta}, so it collapses into W_f, computed once, offline, alongside the
 * centers; the averaged score is one evaluation with the center replaced by mu'.
 *
 * Host function, fp64, synchronous; touches no GPU.
 *   d          head dimension: even, 2 <= d <= 512
 *   theta      rotary base (> 0, finite)
 *   offsets    host int64[n_offsets], the schedule D (e.g. 1, 2, 4, ..., 65536); any values
 *   n_offsets  >= 1
 *   centers    host float[n_units][F][2]: E[q_f] as (re, im), or NULL (then mu_out is not
 *              written and n_units is ignored)
 *   n_units    >= 0
 *   W_out      host double[F][2] (re, im): always written
 *   mu_out     host float[n_units][F][2]: mu' rounded once from fp64 to binary32 (nearest);
 *              may be NULL; written only when centers != NULL
 * Errors: TRI_ERR_ARG for a bad size, theta, or a NULL W_out / offsets.
 */
int tri_fold_weights(int d, double theta, const int64_t* offsets, int n_offsets,
                     const float* centers, int n_units, double* W_out, float* mu_out);

/*
 * tri_score - offset-averaged trigonometric score of every cached key.
 *
 *   score[r] = Re{ sum_f mu'_{u,f} * conj(k_{r,f}) * e^{i omega_f (t_u - pos[r])} }
 *
 * for every row r of unit u. [N] "The same score, read as arrows in the plane" (complex
 * form of the rotary score) and "The averaging step" (the same form with mu' = E[q] W
 * equals the average over the offset schedule). The norm term S_norm of [N] "The score
 * TriAttention computes" is not defined there and is not included.
 *
 *   keys        device, [total_rows][d] elements of `dtype`, rows of unit u at
 *               row_off[u] .. row_off[u+1]-1
 *   dtype       TRI_DT_BF16 or TRI_DT_F32
 *   layout      TRI_BANDS_INTERLEAVED or TRI_BANDS_HALF_SPLIT, optionally | TRI_KEYS_ROTATED
 *   d           64, 128 or 256
 *   theta       rotary base (> 0, finite); the kernel derives omega_f from it
 *   row_off     device int64[n_units+1]: 0 = row_off[0] <= row_off[1] <= ... = total_rows
 *   n_units     >= 1
 *   total_rows  host copy of row_off[n_units] (>= 0)
 *   max_rows    host bound on every N_u (>= 0); rows of a unit beyond it are not scored
 *   pos         device int32[total_rows]: position of each key (not read, and may be NULL,
 *               with TRI_KEYS_ROTATED)
 *   t_now       device int32[n_units]: current position of each unit
 *   mu          device float[n_units][F][2]: mu' (tri_fold_weights' mu_out)
 *   scores      device float[total_rows]: output (binary32); must not overlap the inputs
 *   ws          device workspace or NULL; see below
 *   ws_bytes    in/out, see below
 *   stream      hipStream_t or NULL
 * Workspace protocol (optional radix histogram for tri_select_topb):
 *   ws_bytes == NULL             no workspace: scores only.
 *   ws == NULL, ws_bytes != NULL  query: *ws_bytes = required size; returns TRI_OK, no launch.
 *   both non-NULL                 *ws_bytes must be >= the required size (else
 *                                 TRI_ERR_WORKSPACE). The workspace must be in its rest state
 *                                 (see tri_select_topb; zero-filled once after allocation); the score
 *                                 kernel adds each unit's 12-bit top-digit histogram of the
 *                                 scores into it, and tri_select_topb called with
 *                                 TRI_SELECT_HIST_FROM_SCORE and the same ws consumes it and
 *                                 returns ws to its rest state.
 * Rotated keys (TRI_KEYS_ROTATED): a serving cache that stores keys after the rotary
 *   embedding holds krot_{r,f} = k_{r,f} e^{i omega_f pos[r]}. Rotations compose by adding
 *   angles ([N] "The same score, read as arrows in the plane"), so the same score is
 *       score[r] = Re{ sum_f (mu'_{u,f} e^{i omega_f t_u}) * conj(krot_{r,f}) },
 *   a dot product of each key with one coefficient vector per unit: positions are not read
 *   and no trigonometry is evaluated per key.
 * Device preconditions: 0 <= t_u - pos[r] < 2^24 (rotated keys: 0 <= t_u < 2^24); finite keys
 *   and mu'.
 * Precision: rotation phase in 23-bit fixed point plus a binary32 residual, hardware
 *   sine/cosine, binary32 accumulation; mu' (with rotated keys, mu' e^{i omega t}) enters as a
 *   two-term bfloat16 split for bf16 keys.
 */
int tri_score(const void* keys, int dtype, int layout, int d, double theta,
              const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
              const int32_t* pos, const int32_t* t_now, const float* mu, float* scores,
              void* ws, size_t* ws_bytes, void* stream);

/*
 * tri_score_max - the maximum over the offset schedule instead of the mean.
 *
 *   score[r] = max_{delta in D} Re{ sum_f E[q_{u,f}] * conj(k_{r,f}) * e^{i omega_f (t_u - pos[r] + delta)} }
 *
 * [N] "What it saves, and what it does not": the fold needs the mean over the offsets to be
 * linear and does not cover the variant that takes the maximum over them, so every offset is
 * evaluated. The rotation by the offset is applied to the key's rotated product (rotations
 * compose by adding angles, [N] "The same score, read as arrows in the plane"), so each offset
 * costs two FMAs per band; for d = 128 the offsets are one matrix product per 16 keys, on the
 * matrix cores (bf16 operands split into two terms each, fp32 accumulation).
 *
 * Arguments as in tri_score, except:
 *   offsets     host int64[n_offsets], the schedule D; 0 <= delta < 2^24 each
 *   n_offsets   1 .. 32 (more: TRI_ERR_UNSUPPORTED)
 *   centers     device float[n_units][F][2]: E[q_f] itself (not folded)
 *   layout      TRI_BANDS_INTERLEAVED or TRI_BANDS_HALF_SPLIT, optionally | TRI_KEYS_ROTATED: the keys
 *               were stored after the rotary rotation at their positions; then
 *               conj(k) e^{i omega (t - p + delta)} = conj(k_rot) e^{i omega (t + delta)}, pos is not
 *               read (it may be NULL), and for d = 128 the score is a matrix product of the stored
 *               key rows themselves (no per-key sine or cosine)
 * The workspace protocol is tri_score's: with ws, the histogram of these scores is added for
 * tri_select_topb (TRI_SELECT_HIST_FROM_SCORE), and tri_compact_kv completes the pass (or
 * tri_prune_pass_max, all three in one call).
 * Device preconditions: 0 <= t_u - pos[r] < 2^24 (rotated keys: 0 <= t_u < 2^24); finite keys
 * and centers.
 */
int tri_score_max(const void* keys, int dtype, int layout, int d, double theta, const int64_t* offsets,
                  int n_offsets, const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                  const int32_t* pos, const int32_t* t_now, const float* centers, float* scores, void* ws,
                  size_t* ws_bytes, void* stream);

/*
 * tri_select_topb - keep the B highest-scoring rows of each unit.
 *
 * [N] introduction: when the cache must be trimmed, every key is scored and the
 * highest-scoring ones are kept. [R] chat settings: a KV budget (default 2048, 12000 for
 * chat) bounds the cache. Order: score descending; equal scores keep the lower row index;
 * -0.0 equals +0.0; NaN ranks below every number. Exactly min(B, N_u) rows are kept.
 *
 *   scores    device float[total_rows]
 *   row_off   device int64[n_units+1] (as in tri_score)
 *   n_units   >= 1
 *   total_rows host copy of row_off[n_units]
 *   max_rows  host bound on every N_u; must be < 2^31 (TRI_ERR_ARG); above 2^27 the select
 *             is not implemented (TRI_ERR_UNSUPPORTED)
 *   B         budget per unit, 0 <= B < 2^31
 *   kept_idx  device int32[n_units][B]: the kept rows' local indices (0 .. N_u-1) in
 *             ascending order, then -1 up to B
 *   kept_cnt  device int32[n_units]: min(B, N_u)
 *   ws        device workspace (required), 256-byte aligned, sized by the query below (about
 *             4 bytes per row of max_rows per unit, plus 16 KB per unit); it holds the radix
 *             histograms, per-granule counts and the candidates. Its rest state has the
 *             histograms at zero (zero-filling the whole workspace once after allocation gets
 *             there); every completed call returns it to its rest state. Calls that share a
 *             workspace must not overlap.
 *   ws_bytes  in/out: with ws == NULL, receives the required size (returns TRI_OK, no
 *             launch); otherwise the size of ws (TRI_ERR_WORKSPACE if too small). The size
 *             depends on n_units and max_rows only.
 *   flags     0, or TRI_SELECT_HIST_FROM_SCORE when tri_score has just added the histogram
 *             of these scores (same row_off, max_rows) into ws
 *   stream    hipStream_t or NULL
 * Method: radix select of the B-th largest score per unit (12 + 10 + 10 bits), the last two
 *   digits resolved among the keys of the threshold's top-digit bin; then the kept indices are
 *   written in order. The arrangement depends on the shape, not the result: with 48 units or
 *   more of up to 2^16 rows and at least 384 groups of 64 output slots in all
 *   (n_units * ceil(min(B, max_rows) / 64)), one workgroup per unit; otherwise, with units of up
 *   to 2^18 rows and at most 4096 such groups, a
 *   candidate kernel (1024 rows per workgroup) and one kernel that resolves the threshold and
 *   writes 64 output slots per workgroup; every other shape takes separate candidate,
 *   threshold and output kernels.
 */
int tri_select_topb(const float* scores, const int64_t* row_off, int n_units,
                    int64_t total_rows, int64_t max_rows, int B, int32_t* kept_idx,
                    int32_t* kept_cnt, void* ws, size_t* ws_bytes, unsigned flags,
                    void* stream);

/*
 * tri_compact_kv - dense copy of the kept rows.
 *
 *   K_out[u][j] = K[row_off[u] + kept_idx[u][j]],  V_out and pos_out likewise,
 *   for j < kept_cnt[u]; rows j >= kept_cnt[u] of the outputs are left untouched.
 *
 * [N] introduction: the cache is pruned to the kept entries; [R]: compressed cache entries.
 * A byte copy (bit exact). Out of place: outputs may not overlap inputs (TRI_ERR_ALIAS).
 *
 *   K, V        device, [total_rows][d] elements of `dtype`
 *   pos         device int32[total_rows], or NULL when pos_out is NULL
 *   dtype, d    as in tri_score (d*elem_bytes must be a multiple of 16)
 *   row_off     device int64[n_units+1]; n_units >= 1; total_rows its host copy
 *   kept_idx    device int32[n_units][B], kept_cnt device int32[n_units] (tri_select_topb)
 *   B           >= 0
 *   K_out, V_out  device, [n_units][B][d] elements of `dtype`
 *   pos_out     device int32[n_units][B], or NULL to copy no positions
 *   stream      hipStream_t or NULL
 * Entries of kept_idx outside 0 .. N_u-1 are skipped (their output row is left untouched).
 */
int tri_compact_kv(const void* K, const void* V, const int32_t* pos, int dtype, int d,
                   const int64_t* row_off, int n_units, int64_t total_rows,
                   const int32_t* kept_idx, const int32_t* kept_cnt, int B, void* K_out,
                   void* V_out, int32_t* pos_out, void* stream);

/*
 * tri_prune_pass - one whole pruning pass: tri_score, tri_select_topb and tri_compact_kv fused,
 * same results as calling the three in turn. Three launches for one layer's heads (score with
 * histogram; candidates; threshold with output and row gather) and for 48 units and more of
 * up to 2^16 rows with 384 output groups or more (score; select; row gather); four for the other
 * shapes (score; candidates; threshold; output with row gather), as in tri_select_topb.
 *
 * Arguments are those of the three functions: K (the keys) and V as in tri_compact_kv, the
 * score arguments as in tri_score, B, kept_idx and kept_cnt as in tri_select_topb, K_out /
 * V_out / pos_out as in tri_compact_kv (pos_out may be NULL), ws / ws_bytes as in
 * tri_select_topb (required; same query protocol). Every check of all three runs before the
 * first launch.
 */
int tri_prune_pass(const void* K, const void* V, int dtype, int layout, int d, double theta,
                   const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                   const int32_t* pos, const int32_t* t_now, const float* mu, int B, float* scores,
                   int32_t* kept_idx, int32_t* kept_cnt, void* K_out, void* V_out, int32_t* pos_out,
                   void* ws, size_t* ws_bytes, void* stream);

/*
 * tri_prune_pass_max - the pruning pass with the maximum over the offsets as the score
 * ([N] "What it saves, and what it does not": the variant the fold does not cover): tri_score_max,
 * tri_select_topb on its histogram and tri_compact_kv fused, same results as calling the three in
 * turn, and the same launches as tri_prune_pass with the max-over-offsets score kernel first.
 *
 * Arguments as in tri_prune_pass, except offsets / n_offsets / centers / layout, which are those
 * of tri_score_max (centers: E[q_f] itself; with TRI_KEYS_ROTATED, pos may be NULL when pos_out
 * is NULL). The workspace
 * is tri_prune_pass's (same size query, same rest state). Every check runs before the first
 * launch.
 */
int tri_prune_pass_max(const void* K, const void* V, int dtype, int layout, int d, double theta,
                       const int64_t* offsets, int n_offsets, const int64_t* row_off, int n_units,
                       int64_t total_rows, int64_t max_rows, const int32_t* pos, const int32_t* t_now,
                       const float* centers, int B, float* scores, int32_t* kept_idx, int32_t* kept_cnt,
                       void* K_out, void* V_out, int32_t* pos_out, void* ws, size_t* ws_bytes, void* stream);

/*
 * tri_prune_inplace - the pruning pass on a cache that is pruned where it lives: the steady
 * state of [R] chat serving, where every prefill chunk (1024 tokens with
 * --max-num-batched-tokens 1024) appended to a cache of B kept rows triggers compression back
 * to B (budget 12000 for chat).
 *
 * Scores and selects exactly as tri_prune_pass (same order, ties and counts). Instead of copying
 * the kept rows out, it moves the fewest rows so that unit u's kept rows occupy its first
 * m_u = min(B, N_u) rows: a kept row among the first m_u stays in place; each slot below m_u
 * whose row is dropped receives a kept row from at or beyond m_u - the highest such row goes to
 * the lowest freed slot, the next highest to the next, and so on - with its V row and its
 * position. At most min(m_u, N_u - m_u) rows move; rows from m_u on are left as they were (stale
 * copies). Positions are sparse after the first pass, which the score handles as any others.
 *
 *   K, V        device, [total_rows][d] elements of `dtype`: read and rewritten in place
 *   pos         device int32[total_rows]: read (unless TRI_KEYS_ROTATED) and permuted with the
 *               rows; may be NULL with TRI_KEYS_ROTATED, then no positions are kept
 *   dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, t_now, mu  as in tri_score
 *   B           budget per unit, >= 0
 *   scores      device float[total_rows]: the scores, in the row order before the moves
 *   kept_cnt    device int32[n_units]: m_u
 *   ws, ws_bytes  workspace as in tri_select_topb, with its own size query (it also depends on B)
 *   stream      hipStream_t or NULL
 * Launches: score with histogram; threshold with the freed-slot and mover lists (one
 * workgroup per unit, units up to 2^16 rows; longer: candidates, threshold, lists); moves.
 * No buffer may overlap another (TRI_ERR_ALIAS).
 */
int tri_prune_inplace(void* K, void* V, int32_t* pos, int dtype, int layout, int d, double theta,
                      const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                      const int32_t* t_now, const float* mu, int B, float* scores, int32_t* kept_cnt,
                      void* ws, size_t* ws_bytes, void* stream);

/*
 * tri_prune_pass_noalloc - tri_prune_pass for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call hipMalloc, harnesses that forbid it.
 *
 * Same arguments, checks, results and kernels as tri_prune_pass, without ws / ws_bytes: the
 * workspace is a static device array of TRI_NOALLOC_SCRATCH_BYTES in the library's code object,
 * one per GPU, held from the library's first launch on that GPU until the process ends. The call
 * allocates nothing (no hipMalloc, no allocating library routine). Before the pass it zero-fills
 * the array's histograms with a kernel of its own (one launch more than tri_prune_pass), so it
 * does not depend on what an earlier call left in the array. Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two host threads) race, and the caller
 * must order them.
 *
 *   stream  hipStream_t or NULL; a non-NULL stream must belong to the current device
 * Errors: as tri_prune_pass; TRI_ERR_WORKSPACE, checked first, when the pass needs a workspace
 * larger than TRI_NOALLOC_SCRATCH_BYTES (tri_prune_pass's size query gives the need: about
 * 4 bytes per row of max_rows per unit plus 16 KB per unit, so 64 MiB holds, for example,
 * 288 units of 32768 rows); TRI_ERR_ARG when the stream is on another device; TRI_ERR_HIP when
 * the array's address cannot be obtained.
 */
#define TRI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int tri_prune_pass_noalloc(const void* K, const void* V, int dtype, int layout, int d, double theta,
                           const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                           const int32_t* pos, const int32_t* t_now, const float* mu, int B, float* scores,
                           int32_t* kept_idx, int32_t* kept_cnt, void* K_out, void* V_out, int32_t* pos_out,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_H */
