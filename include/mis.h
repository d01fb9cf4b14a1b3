/*
 * mis.h - C ABI of the multiple-item scoring (MIS) hot path for AMD Instinct
 * MI355X (gfx950 / CDNA4).
 *
 * The method (From Generation to Scoring: Scaling LLM-Based Semantic Labeling
 * at LinkedIn, §4.1, Eq. 3 and Eq. 4): one prefill packs a shared query
 * prefix q and N candidate items c_1..c_N, each closed by a delimiter token
 * (LinkedIn SGLang blog, "Multi-item-scoring" section). Under the MIS mask
 * every prefix token attends causally to the prefix, and every item token
 * attends to the whole prefix plus the earlier tokens of its own item, never
 * to another item. Position ids restart at Lq in every item. The label
 * log-probabilities of an item are read from the next-token logits at its
 * last token (its closing delimiter): one row of K label scores per item, in
 * input order, columns in the requested label order (Scaling JEV-like
 * Decision Models with SGLang, "Getting Started with the Score API").
 *
 * Stream-ordered calls:
 *   mis_build_segments    host metadata -> per-token item/position ids,
 *                         per-item readout positions, per-tile classes
 *   mis_apply_rope        rotary embedding of Q and K at the reused positions
 *   mis_attention_prefill MIS prefill attention (skips fully masked tiles)
 *   mis_attention_append  the same for item rows only, against a cached prefix
 *   mis_score_labels      readout gather -> LM head -> full-vocab logsumexp
 *                         -> label log-probs (mis_score_labels_at: at any
 *                         token rows, e.g. several markers per item)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Return value: MIS_OK (0) or a negative MIS_ERR_* code. On error the
 *   thread-local text of mis_last_error() says what was wrong. All argument
 *   and metadata checks run on the host before anything is enqueued, so a
 *   call that fails its checks has no effect on the device.
 * - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *   Every device write is enqueued on that stream; results are ready once the
 *   stream has been synchronised.
 * - The library never allocates device memory. The caller owns every device
 *   buffer; the *_bytes queries give the sizes. mis_build_segments uploads its
 *   metadata through a small ring of page-locked host slots that the library
 *   allocates once per device and keeps until the process ends.
 * - HIP graph capture: the attention, rotation and scoring calls enqueue
 *   kernels only (no memory sets, copies or host waits), so they can be
 *   captured. mis_build_segments (when its metadata does not fit in the
 *   builder's kernel arguments) and mis_score_labels_at copy from a staging
 *   slot that later calls reuse, so a replay could read another call's data:
 *   run them outside capture. A segment buffer built once serves any number
 *   of captured calls.
 * - Packed ("varlen") token-major layout: request r owns packed tokens
 *   [cu_seqlens[r], cu_seqlens[r+1]); its first prefix_lens[r] tokens are the
 *   prefix, then its items follow back to back in input order. Items are
 *   numbered globally, request by request (row order of the scores).
 * - Integer sizes are int32; every total must fit in int32.
 */
#ifndef MIS_H_
#define MIS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MIS_OK 0
#define MIS_ERR_ARG (-1)         /* null pointer, negative size, Hq % Hkv != 0, ... */
#define MIS_ERR_SEGMENTS (-2)    /* malformed request/item metadata */
#define MIS_ERR_LABEL (-3)       /* K < 1, K > MIS_MAX_LABELS, label id outside [0, V) */
#define MIS_ERR_WORKSPACE (-4)   /* a caller buffer is smaller than its size query */
#define MIS_ERR_UNSUPPORTED (-5) /* shape / dtype / tile combination not compiled */
#define MIS_ERR_HIP (-6)         /* the HIP runtime reported an error (incl. no device) */

#define MIS_MAX_LABELS 256

/* Element type of Q/K/V/O, hidden states and LM head. */
typedef enum { MIS_F32 = 0, MIS_BF16 = 1 } mis_dtype;

/*
 * Segment descriptors, filled by mis_build_segments. Host struct; the
 * pointers are device addresses inside the caller's dev_buf, which must stay
 * alive (and unmodified) for as long as the struct is used.
 */
typedef struct mis_segments {
  int32_t num_requests; /* B */
  int32_t total_tokens; /* T = cu_seqlens[B] */
  int32_t total_items;  /* N */
  int32_t block_m;      /* query-tile height of the tile classes */
  int32_t block_n;      /* key-tile width of the tile classes */
  int32_t num_tiles;    /* sum over requests of ceil(T_r/bm) * ceil(T_r/bn) */
  int32_t num_work;     /* sum over requests of ceil(T_r/bm): query tiles */
  int32_t max_seqlen;   /* max_r T_r */
  int32_t num_visits;   /* sum over the work list of visited key tiles (the tiles with a visible cell) */
  /* per request */
  const int32_t *cu_seqlens;  /* [B+1] packed token offsets */
  const int32_t *prefix_lens; /* [B]   Lq of each request */
  const int32_t *cu_items;    /* [B+1] global item offsets */
  const int32_t *cu_tiles;    /* [B+1] tile offsets into tile_class */
  /* per item */
  const int32_t *item_begin;  /* [N] packed index of the item's first token */
  const int32_t *readout_pos; /* [N] packed index of the item's last token (closing delimiter) */
  /* per token */
  const int32_t *item_id;     /* [T] -1 for prefix tokens, else global item index */
  const int32_t *pos_id;      /* [T] prefix token u -> u; item offset d -> Lq + d */
  /* per tile, request-major then query-tile-major:
     0 = no visible cell, 1 = partly visible, 2 = every in-range cell visible */
  const int8_t *tile_class;   /* [num_tiles] */
  /* per query tile, longest first: {request, query tile, end of the prefix
     key-tile range, first key tile of the own-item range} */
  const int32_t *work;        /* [num_work * 4] */
} mis_segments;

/*
 * Device bytes mis_build_segments needs for this metadata and tile shape.
 * cu_seqlens_h: host [B+1]. Errors: ARG, SEGMENTS (offsets), UNSUPPORTED
 * (block_m / block_n not positive multiples of 16, or above 256).
 */
int mis_segments_bytes(int32_t num_requests, const int32_t *cu_seqlens_h, int32_t total_items,
                       int32_t block_m, int32_t block_n, size_t *bytes);

/*
 * Build the segment descriptors of a packed MIS batch (From Generation to Scoring, §4.1: Eq. 3
 * packing, the reused position-id rule and the Eq. 4 mask; SGLang blog's
 * delimiter-closed items). Per-token ids, readout positions and tile classes
 * are computed by GPU kernels; the host validates the metadata, orders the
 * query tiles longest first and stages everything in the builder kernel's
 * arguments (batches whose staged arrays fit 768 words) or with one copy
 * through pinned host memory.
 *
 * In (host, read before return; the caller may free them afterwards):
 *   cu_seqlens_h[B+1]  non-decreasing, cu_seqlens_h[0] = 0, every T_r >= 1
 *   prefix_lens_h[B]   0 <= Lq_r <= T_r
 *   cu_items_h[B+1]    non-decreasing, cu_items_h[0] = 0, cu_items_h[B] = N
 *   item_starts_h[N]   request-relative item starts: the first item of r
 *                      starts at Lq_r, starts strictly increase inside r, and
 *                      each item ends at the next start (the last at T_r);
 *                      a request with no items must have Lq_r = T_r
 *   block_m, block_n   tile shape of the tile classes; mis_attention_prefill
 *                      requires the shape mis_attention_tile_shape returns
 * Out:
 *   dev_buf/dev_bytes  caller's device buffer, >= mis_segments_bytes
 *   out                host struct, filled on success
 * Errors: ARG, SEGMENTS, UNSUPPORTED, WORKSPACE, HIP.
 */
int mis_build_segments(int32_t num_requests, const int32_t *cu_seqlens_h,
                       const int32_t *prefix_lens_h, const int32_t *cu_items_h,
                       const int32_t *item_starts_h, int32_t block_m, int32_t block_n,
                       void *dev_buf, size_t dev_bytes, mis_segments *out, void *stream);

/*
 * Tile shape (block_m x block_n) that mis_attention_prefill uses for this
 * dtype and head configuration; build the segments with it.
 * Errors: ARG, UNSUPPORTED.
 */
int mis_attention_tile_shape(mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                             int32_t *block_m, int32_t *block_n);

/*
 * MIS prefill attention: O = softmax(scale * Q K^T + M) V per query head,
 * M the Eq. 4 mask of From Generation to Scoring, §4.1 inside each request, no attention across
 * requests. Query head h reads KV head floor(h * hkv / hq) (contiguous GQA
 * groups). Key tiles with no visible cell are never loaded; per-cell masking
 * runs only in partly visible tiles.
 *
 * q [T, hq, D], k and v [T, hkv, D], o [T, hq, D]: device, token-major,
 * contiguous, element type dt (bf16 uses fp32 accumulation and fp32 softmax;
 * P and O are rounded to bf16 to nearest even). softmax_scale <= 0 selects
 * 1/sqrt(D). D must be 64 or 128; hq % hkv == 0. With bf16 every request
 * must satisfy (T_r + 64) * hq * D * 2 < 2^32 bytes (the kernels address a
 * request's rows with 32-bit offsets).
 * Errors: ARG, UNSUPPORTED (D, dt, seg tile shape, or a request beyond that
 * range), HIP.
 */
int mis_attention_prefill(const mis_segments *seg, const void *q, const void *k, const void *v,
                          void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                          float softmax_scale, void *stream);

/*
 * Item rows only, against a cached prefix: the same attention as
 * mis_attention_prefill for every item row (the prefix K/V rows are read as
 * they are in k and v, e.g. kept from an earlier pass over the same prefix),
 * without recomputing the prefix rows (From Generation to Scoring, §4.4: a
 * request that carries part of the items prefills the query again unless
 * its prefix is reused). Arguments, layout and errors as for
 * mis_attention_prefill. On return every item row of o holds its result; a
 * prefix row of o either keeps its old contents or, when its 64-row query tile
 * also holds item rows, is rewritten with the value mis_attention_prefill
 * writes.
 */
int mis_attention_append(const mis_segments *seg, const void *q, const void *k, const void *v,
                         void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                         float softmax_scale, void *stream);

/*
 * Rotary position embedding of Q and K in place, at the segment's position
 * ids (From Generation to Scoring, §4.1's position-id rule: prefix token u at u, the token at
 * offset d inside any item at Lq + d), so each item is rotated as if it
 * followed the prefix alone and MIS equals single-item scoring with the
 * rotation applied. Dims i and i + D/2 (i < D/2) of every head row are turned
 * by pos * theta^(-2i/D): (a, b) -> (a cos - b sin, b cos + a sin); angles in
 * fp64 reduced modulo 2 pi, products in fp32, bf16 results rounded to
 * nearest even.
 *
 * q [T, hq, D] and k [T, hkv, D]: device, token-major, contiguous, element
 * type dt, rewritten in place (call once per batch, before
 * mis_attention_prefill). q may be NULL: then only K is rotated (for the
 * *_rope attention calls, which rotate Q themselves). D must be 64 or 128;
 * theta > 0 (for example 10000 or 1000000). Errors: ARG, UNSUPPORTED, HIP.
 */
int mis_apply_rope(const mis_segments *seg, void *q, void *k, mis_dtype dt, int32_t hq, int32_t hkv,
                   int32_t head_dim, float theta, void *stream);

/*
 * Device bytes of a rotary table for num_positions positions:
 * num_positions x head_dim/2 x 2 floats. Errors: ARG, UNSUPPORTED.
 */
int mis_rope_table_bytes(int32_t num_positions, int32_t head_dim, size_t *bytes);

/*
 * Rotary table for the attention calls that rotate Q while loading it:
 * table[p][i] = (cos, sin) of p * theta^(-2i/D) for p < num_positions and
 * i < D/2, float32 pairs, the same values the rotation of mis_apply_rope
 * computes (same position-id rule: From Generation to Scoring, §4.1). It
 * depends on theta, D and num_positions only, so one table serves every
 * layer and every batch whose position ids stay below num_positions.
 *
 * table: device, at least mis_rope_table_bytes; written on stream. D must be
 * 64 or 128; theta > 0. Errors: ARG, UNSUPPORTED, HIP.
 */
int mis_rope_table(int32_t num_positions, int32_t head_dim, float theta, void *table, size_t table_bytes,
                   void *stream);

/*
 * mis_attention_prefill and mis_attention_append with the rotary embedding of
 * Q applied inside the kernel as Q is loaded: q holds Q before rotation and
 * is not modified; k must already be rotated (mis_apply_rope with q = NULL).
 * The result equals mis_apply_rope on Q and K followed by
 * mis_attention_prefill (or _append), bit for bit, without the pass over Q.
 * rope_table: from mis_rope_table for the same D, with table_positions
 * (its num_positions) >= seg->max_seqlen, so every position id is inside.
 * bf16 only. Other arguments, layout and errors as for mis_attention_prefill;
 * ARG for a missing or short table, UNSUPPORTED for f32.
 */
int mis_attention_prefill_rope(const mis_segments *seg, const void *q, const void *k, const void *v,
                               void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                               float softmax_scale, const void *rope_table, int32_t table_positions,
                               void *stream);
int mis_attention_append_rope(const mis_segments *seg, const void *q, const void *k, const void *v,
                              void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                              float softmax_scale, const void *rope_table, int32_t table_positions,
                              void *stream);

/*
 * Device workspace bytes of mis_score_labels for N items, vocabulary V,
 * K labels, hidden size H and element type dt. Errors: ARG, LABEL.
 */
int mis_score_workspace_bytes(int32_t num_items, int32_t vocab, int32_t num_labels,
                              int32_t hidden, mis_dtype dt, size_t *bytes);

/*
 * Label scores of every item (From Generation to Scoring, §3.3, Eq. 2; JEV post, Score API with
 * label_token_ids and apply_softmax; full-vocabulary normalisation is kept).
 * For item n, h_n = hidden[seg->readout_pos[n]] and z_n = lm_head h_n over
 * the whole vocabulary. Without apply_softmax, scores[n,k] = z_n[label_k] -
 * logsumexp(z_n) (a log-probability <= 0); with apply_softmax, scores[n,:]
 * is the softmax of z_n over the K label ids.
 *
 * hidden [T, H] and lm_head [V, H]: device, row-major, element type dt; only
 * readout rows of hidden are read. label_ids_h: host [K], each in [0, V);
 * duplicates allowed. scores: device float32 [N, K], row n = item n (global
 * input order), column k = label_ids_h[k]; may be NULL when N = 0 (the call
 * then only validates its arguments). ws/ws_bytes: device workspace of
 * at least mis_score_workspace_bytes.
 * Errors: ARG, LABEL, WORKSPACE, UNSUPPORTED (bf16 with H % 32 != 0, or H
 * above 4194304), HIP.
 */
int mis_score_labels(const mis_segments *seg, const void *hidden, int32_t hidden_size,
                     const void *lm_head, int32_t vocab, mis_dtype dt, const int32_t *label_ids_h,
                     int32_t num_labels, int32_t apply_softmax, float *scores, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * Bytes of the scoring workspace the library keeps on each GPU for
 * mis_score_labels_noalloc (16 MiB: the partials of about 1,700 items at a
 * 152K-token vocabulary, 2,000 at 128K).
 */
#define MIS_SCORE_SCRATCH_BYTES (16u << 20)

/*
 * mis_score_labels without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). It computes exactly what
 * mis_score_labels computes, with the same kernels, and keeps the per-tile
 * partials in a device array of MIS_SCORE_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; it calls no device
 * or host allocator. Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller. Nothing in the array needs clearing between
 * calls (each call writes every partial it reads).
 *
 * Arguments as for mis_score_labels, without ws/ws_bytes. Errors: those of
 * mis_score_labels, and WORKSPACE when the call's partials (2 * N *
 * ceil(V/128) + N * K floats, each part rounded up to 256 bytes) exceed
 * MIS_SCORE_SCRATCH_BYTES.
 */
int mis_score_labels_noalloc(const mis_segments *seg, const void *hidden, int32_t hidden_size,
                             const void *lm_head, int32_t vocab, mis_dtype dt, const int32_t *label_ids_h,
                             int32_t num_labels, int32_t apply_softmax, float *scores, void *stream);

/*
 * Label scores at caller-chosen token rows: one row of K label scores for
 * each entry of positions_h, from hidden[positions_h[r]], computed exactly as
 * in mis_score_labels. This serves several readout markers per item (setwise
 * scoring, JEV post's score extraction positions) and graded multi-class
 * labels (From Generation to Scoring, §9: several single-token class labels normalised together,
 * with apply_softmax).
 *
 * positions_h: host [num_rows], each in [0, num_tokens), read before return.
 * hidden [num_tokens, H], lm_head [V, H]: device, element type dt. scores:
 * device float32 [num_rows, K] (may be NULL when num_rows = 0). ws/ws_bytes:
 * device workspace of at least mis_score_workspace_bytes(num_rows, ...); the
 * positions are staged into it through the pinned host ring.
 * Errors: ARG (incl. a position out of range), LABEL, WORKSPACE,
 * UNSUPPORTED, HIP.
 */
int mis_score_labels_at(const int32_t *positions_h, int32_t num_rows, int32_t num_tokens,
                        const void *hidden, int32_t hidden_size, const void *lm_head, int32_t vocab,
                        mis_dtype dt, const int32_t *label_ids_h, int32_t num_labels,
                        int32_t apply_softmax, float *scores, void *ws, size_t ws_bytes, void *stream);

/*
 * Kernel choice of the calling thread, for tests and A/B comparisons (every
 * choice computes the same result). Each call picks its kernel by shape
 * unless a choice is set here; the setting holds for later calls on the same
 * thread until changed, and other threads are not affected.
 *   attention: NULL, "" or "auto" (by shape); "pipe" (pipelined loop, 64 query
 *              rows per wave, 4 heads per workgroup when the GQA group size is a
 *              multiple of 4, else 2); "pipe2" (the same loop, 2 heads per
 *              workgroup); "pipe32" (pipelined loop, 32 rows per wave);
 *              "classic" (plain loop). The pipelined loops need an even GQA
 *              group size: odd group sizes always take the plain loop.
 *   score:     NULL, "" or "auto"; "narrow" (128 vocabulary rows x up to 128
 *              items per workgroup); "wide" (256 rows, item blocks by shape) or
 *              "wide3", "wide4", "wide5", "wide6", "wide8" (that many blocks of
 *              32 items); "persist" or "persist3" .. "persist5" (the 256-row
 *              tiles in persistent workgroups with loader waves; needs
 *              hidden_size >= 128, else the wide tiles). Applies to bf16 with
 *              hidden_size % 64 == 0.
 * Errors: ARG (unknown name; the previous setting stays).
 */
int mis_set_kernel_choice(const char *attention, const char *score);

/*
 * Name of the kernel that mis_attention_prefill launches on this thread for
 * these arguments, e.g. "attn_pipe_kernel<4, 1>" ("" and mis_last_error()
 * set when the arguments are invalid). Static storage; never NULL.
 */
const char *mis_attention_kernel_name(const mis_segments *seg, mis_dtype dt, int32_t hq, int32_t hkv,
                                      int32_t head_dim);

/*
 * Name of the LM-head kernel that mis_score_labels launches on this thread
 * for num_items items of hidden size hidden_size, e.g.
 * "score_persist_kernel<5, 3>" (the combine kernel always follows it). Thread-
 * local storage, valid until the next call on this thread; never NULL.
 */
const char *mis_score_kernel_name(int32_t num_items, int32_t hidden_size, mis_dtype dt);

/* Text of the last error on this thread ("" if none). Never NULL. */
const char *mis_last_error(void);

/* Library version string. */
const char *mis_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIS_H_ */
