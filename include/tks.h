/*
 * tks.h -- C ABI of the MI355X (gfx950) sparse-attention indexer + top-k.
 *
 * The operation (HISA abstract; StreamIndex abstract):
 *   a lightweight indexer with H indexer heads scores every causal key s for
 *   every query t as
 *       I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])
 *   and keeps, per query, the k best key indices.  The flat (DSA-style) form
 *   scans every visible key; the HISA form mean-pools keys into blocks,
 *   scores the pooled representatives, keeps the best blocks and runs the
 *   same token indexer only inside them.  Both emit the same per-query top-k
 *   index set.  Selection is streamed: either over query chunks and key
 *   tiles with a partition-merge of partial top-k lists (a tile never holds
 *   every row's scores of every visible key), or, for one query per
 *   sequence, fused into the scoring pass so that only the promising
 *   candidates of each key segment are written.  No [queries x keys] score
 *   tensor is ever allocated.
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers unless stated; the caller allocates and
 *     owns every buffer, including workspaces (sized by the *_workspace
 *     queries).  The library never allocates device memory.
 *   - All calls are asynchronous on `stream`; inputs must stay alive and
 *     unmodified until the stream reaches the end of the call.
 *   - Layouts are dense row-major as annotated.  q, k and pooled keys are
 *     16-byte aligned; score buffers, idx and vals 4-byte aligned.
 *   - q is bf16 [batch, n_q, heads, dim]; w is fp32 [batch, n_q, heads];
 *     k is bf16 [batch, n_k, dim], or OCP e4m3fn codes [batch, n_k, dim]
 *     with a per-token fp32 scale k_scale [batch, n_k] (key value =
 *     scale * e4m3fn(code), scale >= 0).  Inputs must be finite.
 *   - Visibility: key s is seen by query t iff s <= floor((q_pos0 + t) /
 *     causal_ratio) and s < n_k.  q_pos0 = 0 for prefill, n_k - 1 for one
 *     decode token; causal_ratio > 1 is causality at compressed-key
 *     granularity (one key per causal_ratio positions).
 *   - Output rows hold the min(topk, candidates) best keys ordered by score
 *     descending, then key index ascending (-0 equals +0), then -1 (idx) /
 *     NaN (vals) padding.  This order is a total order, so the result is
 *     unique.
 *   - Supported: 1 <= heads <= 64, dim in {32, 64, 128}, 1 <= topk <= 2048,
 *     HISA block in {32, 64, 128, 256}.  Sizes outside return
 *     TKS_EUNSUPPORTED; malformed arguments return TKS_EINVAL; a workspace
 *     smaller than the query returns TKS_EWORKSPACE; a failed launch returns
 *     TKS_EHIP.  Arguments are checked before anything is launched, and a
 *     non-OK status leaves outputs untouched.  tks_last_error() then gives
 *     a thread-local message.  Device faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - Debugging: with the environment variable TKS_DEBUG_SYNC=1 (read once
 *     per process), every launch is followed by a synchronisation of its
 *     stream and a check of the HIP error state, so an asynchronous kernel
 *     failure is returned (TKS_EHIP) by the call that launched it.  Launches
 *     on a stream being captured into a graph are not synchronised.  The
 *     switch changes no result; it only serialises the host with the GPU.
 */
#ifndef TKS_H
#define TKS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TKS_OK = 0,
    TKS_EINVAL = -1,
    TKS_EUNSUPPORTED = -2,
    TKS_EWORKSPACE = -3,
    TKS_EHIP = -4
} tks_status;

typedef enum { TKS_KEY_BF16 = 0, TKS_KEY_FP8_E4M3FN = 1 } tks_key_dtype;

/* HISA forced blocks: block 0 and the query's local block (the block that
 * holds its last visible key). */
enum { TKS_FORCE_FIRST = 1u, TKS_FORCE_LOCAL = 2u };

typedef struct {
    int32_t batch;        /* independent sequences                         */
    int32_t n_q;          /* queries per sequence                          */
    int32_t n_k;          /* keys per sequence                             */
    int32_t heads;        /* indexer heads H                               */
    int32_t dim;          /* indexer head dimension D                      */
    int32_t q_pos0;       /* position of query 0                           */
    int32_t causal_ratio; /* positions per key (1 = token-level causality) */
    int32_t key_dtype;    /* tks_key_dtype                                 */
} tks_shape;

/* Library version (major * 10000 + minor * 100 + patch). */
int tks_version(void);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* tks_last_error(void);

/*
 * Raw indexer scores of a rectangle of (query, key) pairs -- the tile-sized
 * "materialise" step of the StreamIndex abstract, kept for testing and
 * debugging (the top-k calls below never need it).
 *   scores: fp32 [batch, q_count, k_count]; scores[b, i, j] = I[q_begin + i,
 *   k_begin + j] of sequence b, or -inf where the key is not visible.
 * Requires 0 <= q_begin, q_begin + q_count <= n_q, 0 <= k_begin,
 * k_begin + k_count <= n_k.
 */
int tks_indexer_scores(const tks_shape* shape, const void* q, const float* w, const void* k,
                       const float* k_scale, int32_t q_begin, int32_t q_count, int32_t k_begin,
                       int32_t k_count, float* scores, hipStream_t stream);

/*
 * Flat (DSA-style) indexer top-k over every visible key (HISA abstract:
 * the flat token scan it replaces; StreamIndex abstract: chunked
 * partition-merge top-k).  Query rows are processed in chunks of q_chunk
 * rows; keys in tiles of k_tile keys; each tile's partial top-k is merged
 * into a running per-row list.  q_chunk = 0 / k_tile = 0 pick sizes
 * automatically, and the automatic tile never covers every row and every
 * visible key.
 * With one query per sequence (n_q = 1, decode), dim 128 and both sizes
 * automatic, scoring and selection are fused instead (StreamIndex
 * abstract; the threshold-based Indexer-TopK abstract on the same page:
 * write back only the promising candidates and stay exact): each
 * 4096-key segment (with fp8 keys, each quarter of it that one wave
 * scored) keeps its best candidates above a threshold of its own, a
 * finish pass selects the row's top-k from them and proves the
 * result exact (its k-th best is at least every segment's threshold),
 * and a row that fails the proof (heavily tied or clustered scores) is
 * rescored and selected exactly.  The workspace then holds at most 4096
 * candidates per row, not the row's scores.
 * The result does not depend on q_chunk, k_tile or the form taken.
 *   idx:  int32 [batch, n_q, topk];  vals: fp32 [batch, n_q, topk] or NULL.
 * The workspace size depends only on (shape, topk, q_chunk, k_tile).
 */
size_t tks_topk_flat_workspace(const tks_shape* shape, int32_t topk, int32_t q_chunk,
                               int32_t k_tile);
int tks_topk_flat(const tks_shape* shape, const void* q, const float* w, const void* k,
                  const float* k_scale, int32_t topk, int32_t q_chunk, int32_t k_tile,
                  int32_t* idx, float* vals, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * tks_topk_flat without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a static
 * device array of TKS_STATIC_SCRATCH_BYTES in the library, one per GPU,
 * held until the process ends (its address is looked up on a device's
 * first call).  A call whose workspace (tks_topk_flat_workspace) exceeds
 * it returns TKS_EWORKSPACE before anything is launched.  Nothing is
 * allocated.  Every call on a GPU uses that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must not be
 * issued; calls on one stream are ordered.  Counters the kernels need at
 * zero are cleared by the kernels themselves.  Outputs as tks_topk_flat.
 */
#define TKS_STATIC_SCRATCH_BYTES (16u << 20)
int tks_topk_flat_static(const tks_shape* shape, const void* q, const float* w, const void* k,
                         const float* k_scale, int32_t topk, int32_t q_chunk, int32_t k_tile,
                         int32_t* idx, float* vals, hipStream_t stream);

/*
 * Diagnostic of the fused form: *n_redone (host pointer) receives how many
 * rows of the last tks_topk_flat call that used `workspace` with the same
 * (shape, topk, q_chunk, k_tile) took the exact rescoring path; 0 for the
 * tiled form.  Waits for `stream`.
 */
int tks_topk_flat_redone(const tks_shape* shape, int32_t topk, int32_t q_chunk, int32_t k_tile,
                         const void* workspace, int32_t* n_redone, hipStream_t stream);

/*
 * Top-k of rows of a score matrix that is already in device memory (the
 * selection stage on its own).  Row r holds row_len[r] valid scores at
 * scores + r * row_stride (row_len NULL: n_cols for every row); candidate j
 * of a row is key index j.  Scores must not be NaN.
 *   idx / vals: [n_rows, topk] (vals may be NULL).
 *   workspace: tks_topk_scores_workspace(n_rows, n_cols, topk) bytes, 256-byte
 *   aligned.  It is 0 (and NULL is accepted) unless the rows are fewer than
 *   256 and at least 16384 long; such rows are spread over every CU through
 *   a per-row candidate pool of 32 KiB in the workspace.
 */
size_t tks_topk_scores_workspace(int32_t n_rows, int32_t n_cols, int32_t topk);
int tks_topk_scores(const float* scores, int32_t n_rows, int32_t n_cols, int64_t row_stride,
                    const int32_t* row_len, int32_t topk, int32_t* idx, float* vals,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * HISA block pooling (HISA abstract, stage (1): pooled block
 * representatives): pooled[b, j, :] = bf16 nearest-even rounding of the mean
 * of keys j*block .. j*block+block-1 (fp8 keys dequantised first), summed in
 * double in ascending key order.  Only the n_k / block complete blocks are
 * written.
 *   pooled: bf16 [batch, n_k / block, dim].
 */
int tks_hisa_pool_keys(const tks_shape* shape, const void* k, const float* k_scale,
                       int32_t block, void* pooled, hipStream_t stream);

/*
 * Key-cache append with key compression, fp8 quantisation and block pooling
 * fused (StreamIndex abstract: the indexer reads keys compressed by a ratio
 * m; HISA abstract, stage (1): pooled block representatives).  m is
 * shape->causal_ratio, the key dtype shape->key_dtype, the cache capacity
 * shape->n_k keys per sequence; n_q, heads and q_pos0 are not used.
 *
 * Every sequence's raw key stream already holds raw_len keys; the call
 * appends raw[b, 0 .. n_new) (bf16 [batch, n_new, dim], 16-byte aligned) to
 * each sequence b.  Compressed key j is the bf16 nearest-even rounding of
 * the mean of raw keys m*j .. m*j+m-1 (summed in double in position order);
 * when its last raw key arrives it is written to k (bf16 [batch, n_k, dim]),
 * or for fp8 keys as e4m3fn codes of kc / scale (nearest, ties to even,
 * saturating at 448) with k_scale[b, j] = max_d |kc[d]| / 448 in fp32 (0
 * and zero codes for an all-zero key).  With block > 0, pooled block J
 * (bf16 [batch, n_k / block, dim], the value tks_hisa_pool_keys gives from
 * k) is written when its last compressed key arrives, in the same pass: a
 * decode step never re-reads the cache to keep the pooled keys current.
 *   raw_tail: bf16 [batch, m, dim], caller-owned staging of the raw keys of
 *   a group that is still incomplete after a call; it carries state from
 *   one call to the next and must not be modified in between (NULL allowed
 *   when m = 1).  Its content is not read while raw_len is a multiple of m.
 * Requires raw_len >= 0, n_new >= 0, (raw_len + n_new) / m <= n_k, block 0
 * or a supported HISA block.  Only the completed keys, their scales, the
 * completed pooled blocks and the staging slots are written.  Calls that
 * share raw_tail or overlapping cache slots must be ordered on one stream.
 */
int tks_kv_append(const tks_shape* shape, const void* raw, int32_t n_new, int32_t raw_len,
                  void* raw_tail, void* k, float* k_scale, int32_t block, void* pooled,
                  hipStream_t stream);

/*
 * HISA block selection (HISA abstract, stage (1): score the pooled block
 * representatives with the indexer and discard irrelevant regions).  For
 * query t with local block L (the block holding its last visible key):
 * forced blocks are L (TKS_FORCE_LOCAL) and 0 (TKS_FORCE_FIRST, when
 * L > 0); the complete blocks j < L that are not forced are scored as
 * I_blk[t,j] = sum_h w[t,h] * max(0, q[t,h,:] . pooled[j,:]) and the
 * m_scored best (score desc, block asc) are kept.
 *   blk:      int32 [batch, n_q, m_total], kept blocks ascending, -1 padded.
 *   blk_vals: fp32 same shape or NULL; block score, +inf for forced blocks,
 *             NaN for padding.
 *   m_total must equal m_scored + popcount(force_flags) (1 <= m_total <= 512,
 *   m_scored <= 2048).
 */
size_t tks_hisa_block_select_workspace(const tks_shape* shape, int32_t block, int32_t m_scored);
int tks_hisa_block_select(const tks_shape* shape, const void* q, const float* w,
                          const void* pooled, int32_t block, int32_t m_scored,
                          uint32_t force_flags, int32_t* blk, float* blk_vals, int32_t m_total,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * HISA token refinement (HISA abstract, stage (2): the original indexer
 * applied only within the retained candidate blocks; same top-k interface
 * as the flat scan).  Candidates of query t are the visible keys of the
 * blocks listed in its row of blk (ascending, distinct, -1 entries
 * ignored, as tks_hisa_block_select writes them).  q_chunk = 0 picks the
 * row chunk automatically.
 *   idx / vals: as for tks_topk_flat.
 */
size_t tks_hisa_refine_workspace(const tks_shape* shape, int32_t block, int32_t m_total,
                                 int32_t topk, int32_t q_chunk);
int tks_hisa_refine_topk(const tks_shape* shape, const void* q, const float* w, const void* k,
                         const float* k_scale, int32_t block, const int32_t* blk,
                         int32_t m_total, int32_t topk, int32_t q_chunk, int32_t* idx,
                         float* vals, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Re-layout of the selected rows for the sparse attention that consumes the
 * indices (LongCat Sparse Attention abstract, strategy (1): scattered KV
 * entries are copied into a contiguous, hardware-aligned layout so the
 * consumer reads them with coalesced loads).
 *   kv:  [batch, n_kv, row_bytes] bytes (any row type: bf16 latent KV, keys);
 *   idx: int32 [batch, n_q, topk] (as tks_topk_flat / tks_hisa_refine_topk
 *        write them; -1 = empty slot);
 *   out: [batch, n_q, topk, row_bytes]; out[b, t, j] = kv[b, idx[b, t, j]],
 *        zeros where idx is -1 or outside [0, n_kv).
 * row_bytes must be a positive multiple of 16 (at most 65536); kv and out
 * 16-byte aligned.  The slot order of idx is kept.
 */
int tks_gather_selected(const void* kv, int32_t batch, int32_t n_kv, int32_t row_bytes,
                        const int32_t* idx, int32_t n_q, int32_t topk, void* out,
                        hipStream_t stream);

/*
 * Sparse attention over the selected keys (HISA abstract: the sparse
 * attention consumes the per-query index set and reads only those
 * entries).  The pages give no attention shapes; this form has H query
 * heads over one shared K / V head of width 128:
 *     p_j = softmax over the valid slots j of scale * q[b,t,h,:] . k[b,idx_j,:]
 *     out[b,t,h,:] = sum_j p_j v[b,idx_j,:]
 * Slots with idx = -1 or outside [0, n_kv) are ignored; a row without a
 * valid slot gives zeros.  Scores and the softmax run in fp32, the weights
 * enter P.V as bf16.
 *   q:   bf16 [batch, n_q, heads, 128];  k, v: bf16 [batch, n_kv, 128];
 *   idx: int32 [batch, n_q, topk];        out: fp32 [batch, n_q, heads, 128].
 * heads must be a multiple of 16 (16..128), dim 128, 1 <= topk <= 2048.
 * workspace: tks_sparse_attention_workspace bytes, 256-byte aligned
 * (per-split partial outputs).
 */
size_t tks_sparse_attention_workspace(int32_t batch, int32_t n_q, int32_t heads, int32_t topk);
int tks_sparse_attention(const void* q, const void* k, const void* v, int32_t batch, int32_t n_q,
                         int32_t heads, int32_t dim, int32_t n_kv, const int32_t* idx,
                         int32_t topk, float scale, float* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Kernel timing instrumentation (for benchmarks and profiling).  While
 * enabled, every kernel launch the library makes is bracketed by a pair of
 * HIP events recorded on the launch's stream.  tks_profile_enable(1) clears
 * earlier records.  tks_profile_read() waits for the recorded events and
 * returns the summed duration and launch count of one kernel role:
 *   "score_flat"    -- token scoring of tks_topk_flat / tks_indexer_scores
 *                      (fused form: scoring with the segment filter)
 *   "score_pooled"  -- pooled-block scoring of tks_hisa_block_select
 *   "score_refine"  -- scoring of the kept blocks in tks_hisa_refine_topk
 *                      (prefill: with the refinement plans)
 *   "select_flat"   -- top-k selection of tks_topk_flat (fused form: the
 *                      finish and the repair launch)
 *   "select_pooled" -- block selection of tks_hisa_block_select
 *   "select_refine" -- top-k selection of tks_hisa_refine_topk
 *   "select_scores" -- tks_topk_scores
 *   "pool"          -- tks_hisa_pool_keys
 *   "append"        -- tks_kv_append
 *   "gather"        -- tks_gather_selected
 *   "attend"        -- tks_sparse_attention
 * Returns TKS_EINVAL for an unknown role or NULL outputs.
 */
int tks_profile_enable(int on);
int tks_profile_read(const char* role, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* TKS_H */
