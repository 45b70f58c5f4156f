/* sparsekv.h — C ABI of the MI355X (gfx950) sparse top-k decode step.
 *
 * One decode step of top-k sparse attention over a paged KV history:
 *   score every history key for the current query      (sparsekv_score)
 *   select an exact top-k, lowest index winning ties   (sparsekv_topk)
 *   gather the selected K/V through the slot / block table and run softmax
 *   attention over selected + sink + local tokens      (sparsekv_gather_attend)
 * and ParisKV's compressed-code retrieval variant     (sparsekv_encode,
 *                                                      sparsekv_retrieve).
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Pointers inside the structs and pointer arguments are DEVICE pointers
 *   unless marked (host).  The structs themselves are host memory, read
 *   during the call only.
 * - Every call only enqueues work on `stream` and returns: it never
 *   synchronises, never allocates device memory and keeps no state between
 *   calls.  Outputs are valid once the stream reaches them.  The caller owns
 *   every buffer.  Temporary device memory comes from the caller through
 *   (ws, ws_bytes); sparsekv_workspace_size() tells how much.  A workspace
 *   must be zero-filled once when it is allocated; every call leaves it
 *   zero-filled again (its counters are reset on the device), so it can be
 *   reused by any number of calls that are ordered on one stream.  Calls that
 *   share a workspace must not overlap.
 * - Errors are returned as skv_status; nothing aborts.  Host-visible
 *   arguments are validated (null pointers, sizes, modes, workspace size;
 *   every selecting call requires 1 <= k <= L_max, sparsekv_gather_attend
 *   0 <= k <= L_max, sparsekv_block_select 1 <= K <= L_max / 16).
 *   Device-resident data is NOT validated: table entries must point inside
 *   the pools, token-table slots of live tokens must be unique, and
 *   0 <= lo <= hi <= seq_len <= L_max must hold for every sequence.
 * - bf16 is the IEEE-754 binary32 upper half (uint16 storage).  Products are
 *   accumulated in fp32; outputs are fp32.
 *
 * Storage layouts (skv_kv)
 * ------------------------
 * block == 16, block_table: paged pool [n_blocks][H][16][d], logical token t
 *     of sequence b lives in slot block_table[b][t/16]*16 + t%16
 *     (PagedAttention block table; vToken reading notes, background section);
 *     a negative entry marks an unmapped block, whose 16 tokens are dead.
 * block == 16, token_table: the same pool addressed per token,
 *     slot = token_table[b][t] (-1 = dead token)
 *     (vToken reading notes, section 3.2 token table and section 3.4 Eq. (2)).
 * block == 0: contiguous [B][H][L_max][d].
 * In the pools the row of (slot, head h) starts at element
 *     ((slot/16)*H + h)*16*d + (slot%16)*d.
 * v == NULL means the value is the first d_v dims of the key row (a latent
 * KV shared by all query heads, as in MLA: ECHO-OSDI26 wiki page, problem
 * and motivation).
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_EINVAL = 1,        /* bad argument (null pointer, size, mode) */
  SKV_EUNSUPPORTED = 2,  /* valid but not implemented for this shape / dtype */
  SKV_EWORKSPACE = 3,    /* ws_bytes below sparsekv_workspace_size() */
  SKV_ELAUNCH = 4        /* a kernel launch failed (hipGetLastError) */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

typedef enum {
  SKV_OP_SCORE = 0,
  SKV_OP_TOPK = 1,
  SKV_OP_GATHER_ATTEND = 2,
  SKV_OP_ENCODE = 3,
  SKV_OP_RETRIEVE = 4,
  SKV_OP_SELECT = 5,
  SKV_OP_SELECT_ATTEND = 6,
  SKV_OP_BLOCK_SELECT = 7
} skv_op;

/* Caller-owned KV storage (host struct, device pointers). */
typedef struct {
  const void* k;                /* pool or contiguous keys (dtype)            */
  const void* v;                /* values, same layout as k; NULL => latent   */
  skv_dtype dtype;
  int32_t B, H, d_k, d_v;       /* d_v <= d_k when v == NULL                  */
  int32_t block;                /* 16 (paged / token table) or 0 (contiguous) */
  int32_t L_max;                /* logical capacity per sequence              */
  const int32_t* block_table;   /* [B][L_max/16] or NULL                      */
  const int32_t* token_table;   /* [B][L_max] slot or -1, or NULL             */
  const int32_t* seq_len;       /* [B] logical lengths                        */
  int32_t n_blocks;             /* physical 16-token blocks in the pool
                                   (block == 16), 0 = not given; read only by
                                   the validation (sparsekv_validate, debug
                                   builds)                                    */
} skv_kv;

/* Per-sequence windows (device [B] arrays): candidates for top-k are the live
 * t with lo[b] <= t < hi[b]; the sink is live t < lo[b], the local window is
 * live t >= hi[b] (t < seq_len[b]).  ParisKV close-reading, section 2.5: sink
 * and local regions are attended densely, the region between is searched. */
typedef struct {
  const int32_t* lo;
  const int32_t* hi;
} skv_window;

/* ---------------------------------------------------------------- scoring --
 * scores[b][h][t] = max over the G query heads g of KV head h of
 *                   sum_j q[b][h*G+g][j] * K(b, h, t)[j]
 * for every t < L_max; -inf where t >= seq_len[b] or the token is dead.
 * Raw dot product, no scale (ParisKV close-reading, section 一: s_i = <k_i, q>;
 * ECHO-OSDI26 wiki page: the indexer scores every history key before exact
 * top-k).  With kv = an indexer key cache and G = 1 this is the indexer score.
 *   q       [B][H*G][d_k], same dtype as kv->k
 *   scores  [B][H][L_max] fp32 (written in full)
 * Supports: bf16 (G <= 16, d_k % 32 == 0 uses matrix cores for G >= 2) and
 * f32 (G <= 8); every addressing mode; d_k % 8 == 0. */
skv_status sparsekv_score(const skv_kv* kv, const void* q, int32_t G, float* scores,
                          hipStream_t stream);

/* ------------------------------------------------------------ exact top-k --
 * For each row (b, h) of scores [B][H][L_max]: the k largest finite scores
 * among t in [lo[b], hi[b]), ties broken toward the lower t, -0.0 == +0.0.
 * ECHO-OSDI26 wiki page, observation 5: the final selection is an exact
 * top-k.  Output has set semantics, written in ascending t:
 *   idx   [B][H][k] int32, entries past count[b][h] are -1
 *   count [B][H]    int32 = min(k, number of finite candidates)
 * ws: sparsekv_workspace_size(SKV_OP_TOPK, kv, 0, k, NULL) bytes, where only
 * kv->B, kv->H and kv->L_max are read.  Any L_max (a row of more than 32768
 * scores is read twice more: once to list the keys of the threshold's top
 * 12-bit bin, once to write the selection; a bin of more than 16384 keys is
 * resolved by re-reading the row per radix digit). */
skv_status sparsekv_topk(const float* scores, int32_t B, int32_t H, int32_t L_max,
                         skv_window win, int32_t k, int32_t* idx, int32_t* count, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* sparsekv_score followed by sparsekv_topk (same scores, idx and count), with
 * the top-k's first radix digit (a histogram of the score keys) accumulated
 * inside the score scan instead of a second pass over the scores.
 * ws: sparsekv_workspace_size(SKV_OP_SELECT, kv, G, k, NULL) bytes.
 * Equivalent to sparsekv_score_hist + sparsekv_topk_resume on one ws. */
skv_status sparsekv_select(const skv_kv* kv, const void* q, int32_t G, skv_window win, int32_t k,
                           float* scores, int32_t* idx, int32_t* count, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* The two halves of sparsekv_select, for callers that time or schedule them
 * separately: sparsekv_score_hist is sparsekv_score that also adds the key
 * histogram of the candidates in [lo, hi) into ws (a top-k workspace);
 * sparsekv_topk_resume finishes the exact top-k from that histogram.  They
 * must run in this order on the same scores and ws, with no other top-k call
 * on that ws in between. */
skv_status sparsekv_score_hist(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                               float* scores, void* ws, size_t ws_bytes, hipStream_t stream);
skv_status sparsekv_topk_resume(const float* scores, int32_t B, int32_t H, int32_t L_max,
                                skv_window win, int32_t k, int32_t* idx, int32_t* count,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------ threshold-prefiltered top-k --
 * The k-th largest index score of a decode step moves smoothly from step to
 * step, so an EMA (alpha = 0.5) of the past steps' k-th scores predicts the
 * next one (ECHO-OSDI26 wiki page, observation 3 and core method 3; there it
 * decides what to prefetch, the exact top-k still following the scan).  Here
 * the scan lists the keys that reach the prediction, and the exact top-k is
 * resolved over them when at least k survive; the result is always the exact
 * top-k of sparsekv_topk.
 *
 * sparsekv_score_prefilter: sparsekv_score that also lists, per row (b, h),
 * the candidates t in [lo[b], hi[b]) with score >= thr[b][h] into the top-k
 * workspace (at most 16384 per row; more marks the row as overflowed).
 *   thr  [B][H] fp32 predicted threshold, read; -inf lists every candidate.
 * bf16 keys with d_k in {64, 128, 256} and 1 <= G <= 16 (SKV_EUNSUPPORTED
 * otherwise).  ws: sparsekv_workspace_size(SKV_OP_TOPK, kv, 0, k, NULL)
 * bytes, zero-filled before its first use (the list counters stay zero
 * between calls: sparsekv_topk_prefiltered resets them).
 *
 * sparsekv_topk_prefiltered: after sparsekv_score_prefilter on the same ws,
 * the exact top-k of every row (same results as sparsekv_topk), from the
 * survivors when at least k survived and the window spans at most 131072
 * positions, else from the whole row.  Then
 *   thr[b][h] = alpha kth + (1 - alpha) thr[b][h]   (kth if thr was -inf),
 * kth being the row's k-th largest score (-inf with fewer than k candidates).
 *   used [B][H] int32 (optional, may be NULL): 1 where the survivors sufficed. */
skv_status sparsekv_score_prefilter(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                    const float* thr, float* scores, void* ws, size_t ws_bytes,
                                    hipStream_t stream);
skv_status sparsekv_topk_prefiltered(const float* scores, int32_t B, int32_t H, int32_t L_max,
                                     skv_window win, int32_t k, float* thr, float alpha,
                                     int32_t* idx, int32_t* count, int32_t* used, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------- gather + attention --
 * For each sequence b, KV head h and query head g:
 *   A = {idx[b][h][i] : lo <= idx < hi, live} ∪ {live t < lo} ∪ {live t >= hi}
 *   out[b][h*G+g] = sum_{t in A} softmax_t(scale * q . K_t) V_t
 * ParisKV close-reading, section 一 (paper Eqs. (1)-(3)): softmax is
 * recomputed over the full-precision KV of the chosen set; vToken reading
 * notes, section 3.4 Eq. (2): rows are reached through the slot mapping.
 * Computed as split-k online softmax (per split: running max, sum, weighted
 * values) merged exactly by log-sum-exp.  idx entries of -1 are skipped.
 *   q   [B][H*G][d_k] (kv dtype);  idx [B][H][k] int32 logical positions
 *   out [B][H*G][d_v] fp32; an empty A gives 0.
 * Supports d_k == d_v with: bf16, d = 128, G <= 16 (matrix-core scores);
 * bf16, d = 256, G <= 4; fp32, d = 64, G <= 8; fp32, d = 128, G <= 4
 * (split-k vector path); and the latent case v == NULL, bf16, d_k = 576, d_v = 512, H = 1,
 * G % 16 == 0 (matrix-core path). */
skv_status sparsekv_gather_attend(const skv_kv* kv, const void* q, int32_t G, const int32_t* idx,
                                  int32_t k, skv_window win, float scale, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ fused decode step --
 * One whole sparse decode step: sparsekv_score_hist, then the exact top-k and
 * the gather + attention fused into one kernel, then the split merge.
 * Results equal sparsekv_select followed by sparsekv_gather_attend on the
 * same inputs: scores [B][H][L_max], idx [B][H][k] (ascending, -1 padded),
 * count [B][H] and out [B][H*G][d_v] fp32 (definitions above: ParisKV
 * close-reading, section 一, Eqs. (1)-(3); ECHO-OSDI26 wiki page,
 * observation 5; vToken reading notes, section 3.4 Eq. (2)).
 * Supports bf16 keys and values with d_k == d_v == 128 and 1 <= G <= 8, any
 * L_max.  Fewer than 128 rows longer than 16384 slots with k <= 2048 take
 * the scan that lists segment candidates and one kernel that selects each
 * row from them and attends over it (8 workgroups per row, each finishing
 * the selection and attending an eighth), then the split merge: the exact
 * top-k of the candidates is the row's whenever no key a segment left out
 * could rank among it, else the row is selected from its scores.  Other
 * rows of at most one 32768-slot sweep (L_max <= 32768, or 32765 when L_max
 * is not a multiple of 4) take the fused kernel; longer rows with
 * k <= 4096 take one kernel that selects each row and attends over it: with
 * 128 rows or more one workgroup per row lists the row's candidates itself
 * (one pass over its scores), selects and attends; with fewer, 8 workgroups
 * per row each finish the selection after a slice listing and attend an
 * eighth, then the split merge.  Larger k
 * takes the slice listing, the finish, the split attention and its merge,
 * all inside the same call.  With one
 * query head per KV head (G == 1) a token's score is its attention logit
 * (q . k), so the attention takes it from scores and reads only the value
 * rows.
 * ws: sparsekv_workspace_size(SKV_OP_SELECT_ATTEND, kv, G, k, NULL) bytes,
 * zero-filled before its first use; every call leaves its first region (the
 * key histograms) zero again. */
skv_status sparsekv_select_attend(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                  int32_t k, float scale, float* scores, int32_t* idx,
                                  int32_t* count, float* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* The second half of sparsekv_select_attend, for callers that time or
 * schedule the score scan separately: after sparsekv_score_hist(kv, q, G, win,
 * scores, ws, ...) on the same ws, the exact top-k, gather + attention and
 * split merge (same arguments and results as sparsekv_select_attend; scores
 * is read, not written: for G == 1 it must hold that scan's q . K of this
 * kv, since the attention uses it as the logits).
 * Also the indexer + shared-latent step (ECHO-OSDI26 wiki page, problem and
 * motivation: an indexer scores every key, attention runs over its top-k of
 * a latent KV): kv a latent KV (v == NULL, bf16, d_k = 576, d_v = 512,
 * G in {16, 32, 64, 128}) and the scores and ws left by sparsekv_score_hist
 * of the indexer's own KV, which must have the same B, H and L_max.  Rows
 * longer than 32768 slots with k <= 4096 finish the exact top-k inside the
 * attention kernel after one listing pass (every attending workgroup
 * resolves its row's selection from the list); others take the top-k first.
 * ws: sparsekv_workspace_size(SKV_OP_SELECT_ATTEND, kv, G, k, NULL) bytes
 * (for the latent KV), and at least the scoring call's size. */
skv_status sparsekv_select_attend_resume(const skv_kv* kv, const void* q, int32_t G,
                                         skv_window win, int32_t k, float scale,
                                         const float* scores, int32_t* idx, int32_t* count,
                                         float* out, void* ws, size_t ws_bytes,
                                         hipStream_t stream);

/* The indexer + shared-latent decode step in one call (ECHO-OSDI26 wiki
 * page, problem and motivation: a separate indexer key cache scores every
 * history token, and attention over the latent KV runs on the indexer's
 * top-k only): scores[B][H][L_max] = max over the iG indexer heads of
 * iq . ikey (as sparsekv_score on ikv), idx / count = the exact top-k of
 * each row's window by those scores (ascending positions, ties to the lower
 * position, -1 padded), out[B][H*G][512] = the latent attention of the G
 * query heads q over the selected tokens plus sink and local (as
 * sparsekv_gather_attend on kv).  Results equal sparsekv_score_hist(ikv, iq,
 * iG, ...) followed by sparsekv_select_attend_resume(kv, q, G, ...).
 * ikv: the indexer's keys (bf16, d_k in {64, 128, 256}; v unused); kv: the
 * latent KV (v == NULL, bf16, d_k = 576, d_v = 512, G in {16, 32, 64, 128});
 * both with the same B, H and L_max, and the same table layout per
 * sequence.  Rows longer than 32768 slots with k <= 2048 take the scan that
 * lists segment candidates and the latent attention kernel that selects
 * from them (3 kernels with the merge); others take the histogram scan and
 * the resume path.
 * ws: sparsekv_workspace_size(SKV_OP_SELECT_ATTEND, kv, G, k, NULL) bytes,
 * zero-filled before its first use (the histogram path leaves its first
 * region zero again).  Errors: SKV_EINVAL for null pointers, k outside
 * [1, L_max], a non-latent kv or mismatched shapes; SKV_EUNSUPPORTED for
 * other shapes or dtypes; SKV_EWORKSPACE for a short ws. */
skv_status sparsekv_indexer_attend(const skv_kv* ikv, const void* iq, int32_t iG,
                                   const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                   int32_t k, float scale, float* scores, int32_t* idx,
                                   int32_t* count, float* out, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* The two halves of sparsekv_select_attend and sparsekv_indexer_attend on
 * long rows, for callers that time or schedule the score scan separately
 * (as sparsekv_score_hist and sparsekv_select_attend_resume are on the
 * histogram path).  sparsekv_segments(akv, aG, k) is the number of scan
 * segments per row the pair uses when the selecting half attends over akv
 * with aG query heads and top-k k -- k <= 2048 and a selecting kernel that
 * supports the shape: fewer than 128 rows longer than 16384 slots for a GQA
 * akv, rows longer than 32768 slots for a latent one -- or 0 when the pair
 * does not apply (then use the histogram path).
 * sparsekv_score_segments(kv, q, G, win, k, scores, ws, ...): scores
 * [B][H][L_max] as sparsekv_score, and in ws, per row, the candidates of
 * each of its segments: the segment's highest window keys that fit its
 * share of 8192 slots (whole top histogram bins, in position order), their
 * count, and a cut that every key left out lies below (ECHO-OSDI26 wiki page,
 * observation 5: the selection must stay exact).  kv is the scored KV (the
 * indexer's for the latent step) with the same B, H, L_max as akv.
 * sparsekv_select_attend_segments(akv, q, aG, win, k, scale, scores, ...):
 * the exact top-k of each row from those candidates when no cut lies above
 * the k-th of them and no segment left keys out while fewer than k were
 * listed (else that row is selected from its scores alone), then the gather
 * + attention and the split merge; results as sparsekv_select_attend (GQA)
 * or sparsekv_select_attend_resume (latent akv).  Nothing in ws needs to
 * be zero for either call, and they leave the histogram region as they find
 * it.  ws: sparsekv_workspace_size(SKV_OP_SELECT_ATTEND, akv, aG, k, NULL).
 * Errors: SKV_EINVAL for null pointers or k outside [1, L_max];
 * SKV_EUNSUPPORTED where sparsekv_segments is 0 (or the scan's shape is
 * not supported); SKV_EWORKSPACE for a short ws. */
int32_t sparsekv_segments(const skv_kv* akv, int32_t aG, int32_t k);
skv_status sparsekv_score_segments(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                   int32_t k, float* scores, void* ws, size_t ws_bytes,
                                   hipStream_t stream);
skv_status sparsekv_select_attend_segments(const skv_kv* akv, const void* q, int32_t aG,
                                           skv_window win, int32_t k, float scale,
                                           const float* scores, int32_t* idx, int32_t* count,
                                           float* out, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* sparsekv_select_attend for callers that cannot allocate device memory or
 * hand in a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results as
 * sparsekv_select_attend, with the workspace taken from a scratch area the
 * library holds on each GPU it runs on (16 MiB, a device global, kept until
 * the process ends).  The call allocates nothing; it zero-fills the part of
 * the scratch that must start at zero, so no state carries over from an
 * earlier call.  It needs sparsekv_select_attend_noalloc_bytes(kv, G) bytes
 * of scratch (B H 16 KiB of histograms, rounded to 256 bytes, plus
 * B H G 8 (d_v + 2) 4 bytes of split partials) and returns SKV_EWORKSPACE
 * when that exceeds 16 MiB.  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (different streams without
 * ordering between them) race and must not be issued.  Arguments, supported
 * shapes and other errors as sparsekv_select_attend. */
size_t sparsekv_select_attend_noalloc_bytes(const skv_kv* kv, int32_t G);
skv_status sparsekv_select_attend_noalloc(const skv_kv* kv, const void* q, int32_t G,
                                          skv_window win, int32_t k, float scale, float* scores,
                                          int32_t* idx, int32_t* count, float* out,
                                          hipStream_t stream);

/* -------------------------------------------------- block-summary scoring --
 * OasisKV reading notes, section 3.2 (after Quest): each logical 16-token
 * block keeps, per KV head, the coordinate-wise minimum mn and maximum mx of
 * its live keys; a query ranks the blocks from these summaries alone (1/8 of
 * the key bytes of a full scan) and the top K blocks per KV head are
 * attended.  The page gives no score formula; this library takes Quest's
 * upper bound of q . k over the block, max over the G query heads of
 *   sum_i max(q_i mn_i, q_i mx_i) = [max(q,0), min(q,0)] . [mx, mn].
 *
 * Summary pool (caller-owned, bf16): the summary of physical block p, KV head
 * h is the 2 d_k-wide row [mx, mn] at element
 *   ((p/16)*H + h)*16*2*d_k + (p%16)*2*d_k,
 * i.e. a pool of ceil(n_blocks/16) 16-row blocks of width 2 d_k;
 * sparsekv_block_summary_bytes(n_blocks, H, d_k) bytes.  Rows of blocks no
 * call has summarised are never read.
 *
 * sparsekv_block_summarize: (re)builds the summaries of logical blocks
 * j0 <= j < j1 of sequence b (every KV head) from the keys: the block's live
 * tokens are 16 j <= t < min(16 j + 16, seq_len[b], L_max); blocks with no
 * such token or a negative table entry are skipped.  Call it for the blocks
 * whose tokens changed (while decoding: the last block) before the next
 * sparsekv_block_select.  Requires a bf16 paged pool with a block table and
 * d_k in {32, 64, 128}.
 *
 * sparsekv_block_summarize_last: the same for the block holding token
 * min(seq_len[b], L_max) - 1 of every sequence b (none where that is -1): the
 * one block a decode step's appended token changes, all sequences in one
 * launch.
 *
 * sparsekv_block_select: first brings the summary of the block holding each
 * sequence's last token up to date (as sparsekv_block_summarize_last, so a
 * decode step that appended one token per sequence needs no separate
 * summary call; summ is written there only), then for every row (b, h),
 *   blk_scores [B][H][L_max/16] fp32: the bound above for blocks holding a
 *                live token, -inf elsewhere (written in full);
 *   blk_idx    [B][H][K] int32: the K best blocks among those lying wholly
 *                inside [lo[b], hi[b]) (block ceil(lo/16) up to but excluding
 *                floor(hi/16)), exact, ties to the lower block, ascending,
 *                -1 padded;  blk_count [B][H] = min(K, finite candidates);
 *   tok_idx    [B][H][16 K] int32: token 16 blk_idx[u] + e of every chosen
 *                block u, at 16 u + e, -1 where the token is not live or
 *                u >= blk_count -- the idx argument (k = 16 K) of
 *                sparsekv_gather_attend with the same window, which adds the
 *                sink and local tokens.
 *   q [B][H*G][d_k] bf16.  Requires bf16 keys in a block-table pool,
 *   d_k in {32, 64, 128}, 1 <= G <= 16, L_max % 256 == 0.
 * ws: sparsekv_workspace_size(SKV_OP_BLOCK_SELECT, kv, G, K, NULL) bytes,
 * zero-filled before its first use (every call leaves it so). */
size_t sparsekv_block_summary_bytes(int32_t n_blocks, int32_t H, int32_t d_k);
skv_status sparsekv_block_summarize(const skv_kv* kv, int32_t b, int32_t j0, int32_t j1,
                                    void* summ, hipStream_t stream);
skv_status sparsekv_block_summarize_last(const skv_kv* kv, void* summ, hipStream_t stream);
skv_status sparsekv_block_select(const skv_kv* kv, void* summ, const void* q, int32_t G,
                                 skv_window win, int32_t K, float* blk_scores, int32_t* blk_idx,
                                 int32_t* blk_count, int32_t* tok_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------ token-table compaction --
 * vToken reading notes, sections 3.2-3.5 and 4.6.  Token-level eviction
 * leaves holes in the pool's blocks (the intra-block waste ratio of Eq. (1),
 * F = 1 - sum_i n_i / (N S), S = 16); lazy compaction packs the live tokens
 * of a sequence's emptiest private blocks into fewer free blocks, in logical
 * order, and frees the sources.  Planning works on a host copy of the token
 * table (the page keeps the canonical table on the CPU); the copy, the
 * table update and the invariant checks run on the GPU. */
typedef struct {
  int32_t b;                    /* sequence                                   */
  int32_t t;                    /* logical token                              */
  int32_t src, dst;             /* slots before and after the move            */
} skv_move;

/* Eq. (1) over n blocks with n_live[i] live tokens each (host, no GPU). */
double sparsekv_waste_ratio(const int32_t* n_live, int32_t n);

/* Relocation plan for sequence b (host only; no GPU work).
 *   token_table [B][L_max], seq_len [B]: HOST copies; slots < n_blocks * 16.
 *   counts      [n_blocks] live tokens per block over every sequence (host,
 *               the caller's running counts), or NULL to count them here.
 *   free_blocks [n_free] free blocks (host), consumed in this order; n_free
 *               is what the plan may take (free pool + evacuation headroom).
 * Stage 1: F over the blocks holding the sequence's live tokens must exceed
 * theta_F (the page's default is 0.25).  Stage 3: the candidates are the
 * sequence's private blocks (every live token in them is its own) that are
 * not full, emptiest first (ties: lower block), at most max_src; while they
 * would not free strictly more blocks than the ceil(T_live / 16) targets they
 * fill, or need more than n_free targets, the fullest is dropped (stage 2 and
 * invariant I4).  Output (host): moves [n_moves] (room for 16 * max_src), in
 * ascending t, move i going to slot free_blocks[i / 16] * 16 + i % 16;
 * src_blocks [n_src] the freed blocks (ascending); n_dst = targets used.
 * n_moves = 0 when no plan passes.  SKV_EINVAL on a slot outside the pool, or
 * on a free block outside [0, n_blocks), holding a live token (counts[p] > 0)
 * or listed twice among the first n_free entries. */
skv_status sparsekv_compact_plan(const int32_t* token_table, const int32_t* seq_len, int32_t B,
                                 int32_t L_max, int32_t n_blocks, const int32_t* counts, int32_t b,
                                 const int32_t* free_blocks, int32_t n_free, double theta_F,
                                 int32_t max_src, skv_move* moves, int32_t* n_moves,
                                 int32_t* src_blocks, int32_t* n_src, int32_t* n_dst);

/* apply_moves with its copy: for every move (device array), the K row (and
 * the V row when kv->v is set) of every head is copied from slot src to slot
 * dst, then token_table[b][t] = dst.  WRITES kv->k, kv->v and
 * kv->token_table (their const in skv_kv notwithstanding).  Readers ordered
 * after the call on the stream see the moved tokens; the source slots keep
 * their bytes until the caller reuses their blocks.  Requires a token-table
 * pool (block = 16) of n_blocks blocks with rows a multiple of 16 bytes;
 * destination slots must be distinct and hold no live token.  A move with
 * b outside [0, B), t outside [0, L_max) or src / dst outside
 * [0, 16 n_blocks) is skipped -- nothing is read or written for it -- and
 * counted into *err (device int32, added to; may be NULL). */
skv_status sparsekv_compact_apply(const skv_kv* kv, int32_t n_blocks, const skv_move* moves,
                                  int32_t n_moves, int32_t* err, hipStream_t stream);

/* Invariant I1 check (section 4.6: the retained token ids and their K/V
 * contents hashed before and after a migration; the page names no hash).
 * For each sequence b:
 *   hash[b]  = sum mod 2^64 over live t, heads h, rows r (0 = K, 1 = V when
 *              v is stored; R rows), 64-bit words w_j of the stored row
 *              (32-bit words 2j, 2j + 1, low first) of
 *              mix64((s + (j + 1) * 0x9e3779b97f4a7c15) ^ w_j),
 *              s = mix64((t H + h) R + r),
 *   count[b] = live tokens,
 * mix64 being the SplitMix64 finaliser (Steele, Lea, Flood 2014).  The hash
 * does not depend on where tokens are stored.  hash, count: device [B].
 * Rows of a multiple of 16 bytes, at most 4 KB; SKV_EUNSUPPORTED otherwise. */
skv_status sparsekv_live_hash(const skv_kv* kv, uint64_t* hash, int32_t* count,
                              hipStream_t stream);

/* Invariant I2 check over every sequence of a paged or token-table pool of
 * n_blocks blocks: result[0] = live tokens whose slot another live token
 * already claims, result[1] = live tokens whose slot is outside the pool
 * (device int32 [2]).  ws: sparsekv_check_unique_ws_bytes(n_blocks) bytes
 * (any content; it is rewritten by every call). */
size_t sparsekv_check_unique_ws_bytes(int32_t n_blocks);
skv_status sparsekv_check_unique(const skv_kv* kv, int32_t n_blocks, int32_t* result, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------- compressed-code retrieval --
 * ParisKV close-reading, sections 2.2-2.5: keys and the query are normalised
 * and rotated by one SRHT R = H_d diag(signs) / sqrt(d); each of n_sub
 * subspaces of m = 8 dims stores the id of its sign-pattern centroid
 * (2^m = 256 fixed centroids), a 4-bit code per coordinate (1 sign bit + 3
 * magnitude bits from Lloyd-Max levels) and a correction weight
 * w = |k| r_b / <v_b, u_b>. */
typedef struct {                /* host struct */
  int32_t d, n_sub, m;          /* d = n_sub * m; supported: d = 128, m = 8  */
  const int8_t* signs;          /* device [d], +1 / -1                        */
  float levels[8];              /* magnitude reconstruction values, ascending */
  float thresh[7];              /* |u| >= thresh[i] moves past level i        */
} skv_codebook;

typedef struct {                /* host struct, device arrays */
  uint8_t* ids;                 /* [H][cap][n_sub] centroid id per subspace   */
  uint32_t* cw;                 /* [H][cap][n_sub][2]: per subspace its codes
                                   word (coordinate c of the subspace in bits
                                   4c..4c+3: sign bit 3, magnitude bits 0-2)
                                   then its correction weight w (fp32 bits);
                                   an entry's 16 pairs fill one 128-byte line,
                                   so the rerank reads one line per candidate */
  int32_t* hist;                /* [H][n_sub][256] entries per centroid       */
  int32_t* pos;                 /* [cap] logical position of each entry       */
  int32_t n, cap, H;            /* n entries in use (host-side count)         */
} skv_index;

/* Fill the codebook's levels / thresholds: the library's own Lloyd-Max fixed
 * point (float64, rounded once to fp32) for |u_j| with (u_j)^2 ~
 * Beta(1/2, (m-1)/2) (ParisKV close-reading, section 2.4, Prop. 4.1).
 * Host only; m in [3, 16]. */
skv_status sparsekv_codebook_init(int32_t m, float levels[8], float thresh[7]);

/* Append the keys at logical positions [t0, t1) of sequence b (contiguous or
 * block-table kv, bf16, d_k == cb->d) of every KV head to the index as
 * entries [index->n, index->n + t1 - t0); adds their ids to index->hist
 * (which the caller zeroes once when the index is created) and advances the
 * host-side index->n.  Fails with SKV_EINVAL if the index would overflow. */
skv_status sparsekv_encode(const skv_codebook* cb, const skv_kv* kv, int32_t b, int32_t t0,
                           int32_t t1, skv_index* index, hipStream_t stream);

/* Update buffer of the compressed path (ParisKV close-reading, section 2.5).
 * The history of sequence b is laid out as
 *   Sink [0, sink) | Retrieval [sink, sink + index->n) (encoded in the index)
 *   | Local (`local` tokens) | Update buffer (the newest tokens)
 * and Sink, Local and the buffer are attended densely.  New tokens enter the
 * buffer; when it holds `update` tokens they join Local, and the `update`
 * oldest Local tokens are encoded into the index (the page amortises index
 * updates this way, with update = 256 or 512).  Call this after appending
 * tokens, with the sequence's new length seq_len (host value; the device
 * seq_len[b] must already hold it): it applies the rule for every full buffer
 * (seq_len - sink - index->n >= local + update), appending the tokens
 * [sink + index->n, sink + index->n + f * update) as sparsekv_encode does, and
 * writes f to *flushed (host, may be NULL).  The retrieval window for
 * sparsekv_gather_attend is then lo = sink, hi = sink + index->n.  The index
 * must hold exactly positions [sink, sink + index->n) of sequence b.
 * Errors as sparsekv_encode; SKV_EINVAL also when seq_len < sink + index->n
 * or update < 1 (nothing is encoded then). */
skv_status sparsekv_update_buffer(const skv_codebook* cb, const skv_kv* kv, int32_t b,
                                  int32_t seq_len, int32_t sink, int32_t local, int32_t update,
                                  skv_index* index, int32_t* flushed, hipStream_t stream);

/* Optional intermediate outputs of a retrieval (device arrays, NULL = skip). */
typedef struct {
  uint8_t* votes;               /* [H][n] collision score S_i (0..6*n_sub)   */
  int32_t* cand;                /* [H][C] candidate entry numbers, ascending  */
  float* est;                   /* [H][C] rerank estimate of each candidate   */
} skv_retrieve_trace;


/* Collision vote + bucket top-C + 4-bit rerank + exact top-k_final for the
 * index entries [0, index->n) of every KV head (ParisKV close-reading,
 * sections 2.3-2.5):
 *   1. the query heads are normalised and rotated like the keys; per
 *      subspace the 256 centroids are ranked by similarity (ties: lower id)
 *      and, walking that ranking with the exclusive prefix count P of the
 *      index histogram, a centroid gets tier weight 7 - l for the smallest
 *      l with P < T_l (0 if P >= T_rho), T_rho = ceil(rho n),
 *      T_l = ceil(p_l T_rho), p = .05 .15 .30 .50 .75 1.0 (float64, host);
 *   2. S_i = max over the G query heads of sum_b weight[b][id_ib];
 *   3. the C = min(n, ceil(beta n)) largest S_i, ties to the lower entry;
 *   4. est_i = max_g |q_g| sum_b w_ib <v_ib, q~_gb> (fp32, tree sums);
 *   5. the k_final largest est_i, ties to the lower entry.
 *   q      [H*G][d] bf16 query heads (G per KV head, G <= 4)
 *   idx    [H][k_final] int32 logical positions (index->pos of the winners),
 *          ascending; -1 past n_cand
 *   n_cand [H] int32 = min(k_final, C)
 * Requires rho >= beta > 0, d = 128, m = 8.
 * ws: sparsekv_retrieve_workspace_size(index, G, beta, k_final) bytes for the
 * largest index->n it will serve, zero-filled once; the regions kept zero
 * between calls sit at fixed offsets, so an index that grows between calls
 * (sparsekv_update_buffer) keeps its workspace. */
skv_status sparsekv_retrieve(const skv_codebook* cb, const skv_index* index, const void* q,
                             int32_t G, double rho, double beta, int32_t k_final, int32_t* idx,
                             int32_t* n_cand, const skv_retrieve_trace* trace, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ validation --
 * Checks of the device-resident data the other calls take on trust (vToken
 * reading notes, section 3.5 invariant I2: every live token maps to a valid
 * slot inside the pool and no two live tokens to one slot; section 4.6 checks
 * the invariants around every migration), OR-ed into flags[0] (device int32):
 *   SKV_FLAG_BAD_SEQ_LEN  seq_len[b] outside [0, L_max]
 *   SKV_FLAG_BAD_WINDOW   not 0 <= lo[b] <= hi[b] <= seq_len[b] (win given)
 *   SKV_FLAG_BAD_SLOT     a mapping of a token t < seq_len[b] that is neither
 *                         -1 nor a valid slot (token table: < -1 or
 *                         >= 16 n_blocks; block table: < -1 or >= n_blocks;
 *                         the upper bounds only when kv->n_blocks > 0)
 *   SKV_FLAG_DUP_SLOT     two live tokens share a slot (token table) or two
 *                         logical blocks a physical block (block table);
 *                         only when kv->n_blocks > 0
 *   SKV_FLAG_BAD_IDX      an idx entry outside [-1, L_max)
 *   SKV_FLAG_DUP_IDX      an idx row names a position twice
 * Reads seq_len, the table, win.lo / win.hi (both NULL: not checked) and
 * idx [B][H][k] (NULL: not checked); never the K/V pools, so invalid tables
 * form no address into them.  kv->k / kv->v are not read.
 * ws: sparsekv_validate_ws_bytes(kv, k) bytes (any content).
 *
 * Builds compiled with SKV_DEBUG run the same checks at the start of every
 * call that reads tables, windows or selected positions, into a flag word
 * the library holds per device; sparsekv_debug_status synchronises the
 * device, returns that word in *flags (host) and clears it (SKV_EUNSUPPORTED
 * and 0 in release builds).  Debug builds allocate their check workspace with
 * hipMalloc, so their calls must not be captured in a graph; the checks
 * report, they do not stop the call that follows them. */
enum {
  SKV_FLAG_BAD_SEQ_LEN = 1,
  SKV_FLAG_BAD_WINDOW = 2,
  SKV_FLAG_BAD_SLOT = 4,
  SKV_FLAG_DUP_SLOT = 8,
  SKV_FLAG_BAD_IDX = 16,
  SKV_FLAG_DUP_IDX = 32
};
size_t sparsekv_validate_ws_bytes(const skv_kv* kv, int32_t k);
skv_status sparsekv_validate(const skv_kv* kv, skv_window win, const int32_t* idx, int32_t k,
                             int32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);
skv_status sparsekv_debug_status(int32_t* flags);
int32_t sparsekv_is_debug_build(void);

/* Workspace bytes for an op.  Arguments an op does not use may be NULL / 0:
 *   SCORE, ENCODE: 0;   TOPK, SELECT: kv->B, kv->H, kv->L_max;
 *   BLOCK_SELECT: kv, G (K is not read);
 *   GATHER_ATTEND: kv, G, k;   RETRIEVE: index, G, k (= k_final) with
 *   beta = 1 (an upper bound); sparsekv_retrieve_workspace_size() takes the
 *   actual beta. */
size_t sparsekv_workspace_size(skv_op op, const skv_kv* kv, int32_t G, int32_t k,
                               const skv_index* index);
size_t sparsekv_retrieve_workspace_size(const skv_index* index, int32_t G, double beta,
                                        int32_t k_final);

const char* sparsekv_status_string(skv_status s);
int32_t sparsekv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEKV_H */
