/*
 * infllmv2.h -- C ABI of an MI355X (gfx950) library for InfLLM v2 block-sparse
 * attention: semantic-kernel pooling, block scoring, top-K block selection, and
 * sparse (prefill, decode, draft-tree) and dense attention.
 *
 * The method (MiniCPM4 technical-report summary, QbitAI repost, section
 * "Model architecture: InfLLM v2 native sparse attention"): the context is cut
 * into fixed-size blocks; each block is represented by several fine-grained
 * "semantic kernels"; a query's relevance to a block is the maximum of its
 * relevance to the kernels the block contains (item 1); the query heads of
 * one GQA group share one set of blocks (item 2); attention then runs over the
 * selected blocks only, and short contexts keep dense attention. Tree-draft
 * verification uses the same sparse kernel with a local attention mask stored
 * as packed bits (same summary, section on fusing speculative sampling,
 * quantization and long-context algorithms).
 *
 * Fixed readings used throughout (the pages leave them open):
 *   - block_size 64; kernels are the means of 32-key windows at stride 16 that
 *     lie inside a block (3 per block), rounded to bf16 (nearest even);
 *   - block score R(j) = sum over the group's query heads of the max over
 *     block j's kernels of the raw dot product q . kbar (no scaling);
 *   - a query at absolute position p has candidates j < floor(p/64) (complete
 *     blocks before its own block); its own block floor(p/64) is always
 *     attended, causally, on top of the K selected blocks;
 *   - top-K keeps the K highest scores (compared in fp32), the lower block
 *     index first on equal scores; the output row is ascending and padded
 *     with -1 when there are fewer than K candidates (then all are taken);
 *   - a query row with fewer than dense_threshold visible keys attends all of
 *     them; dense_threshold 0 disables the rule;
 *   - softmax scale 1/sqrt(head_dim) unless given; bf16 outputs are rounded
 *     to nearest even; lse is the natural log of the softmax denominator.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as device pointers to raw 16-bit patterns;
 *     all pointers are device pointers unless stated; all tensors are dense,
 *     row-major, 16-byte aligned;
 *   - layouts: q   [B][Hq][n_q][D]         (heads g*G .. g*G+G-1 form group g)
 *              k,v [B][Hkv][kv_cap][D]     (rows >= kv_len are never read)
 *              kbar [B][Hkv][T][3][D/8][32][8]  nblk = ceil(kv_cap / 64),
 *                                          T = ceil(nblk / 32): kernel m of block j,
 *                                          elements 8p .. 8p+7, sit at
 *                                          [b][g][j/32][m][p][j%32][0..7] (tiles of 32
 *                                          blocks; in a tile the 32 copies of one
 *                                          16-byte piece are adjacent). The buffer
 *                                          holds whole tiles: entries of blocks
 *                                          >= nblk are read but never affect a result
 *              scores [B][Hkv][n_q][nblk]  fp32, -inf past a row's candidates
 *              idx [B][Hkv][n_q][K]        int32
 *              out [B][Hq][n_q][D]         bf16
 *              lse [B][Hq][n_q]            fp32, optional (NULL: not written)
 *              tree_mask [B][n_q]          uint64
 *   - the caller owns every buffer; the library allocates nothing, keeps no
 *     pointer after returning, and takes scratch memory only as an explicit
 *     workspace argument;
 *   - `stream` is a hipStream_t (NULL = the default stream); each call checks
 *     its arguments on the host, enqueues its kernels and returns without
 *     synchronizing; calls on different streams may run from different threads;
 *   - return value: 0 on success or a negative INFLLMV2_* status. Argument
 *     checks run before any HIP call, so a rejected call launches nothing.
 *     infllmv2_last_error() (per thread) describes the last failure.
 */
#ifndef INFLLMV2_H
#define INFLLMV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define INFLLMV2_API __attribute__((visibility("default")))
#else
#define INFLLMV2_API
#endif

#define INFLLMV2_OK 0
#define INFLLMV2_INVALID_ARGUMENT (-1)   /* null pointer, bad shape, misaligned pointer */
#define INFLLMV2_UNSUPPORTED (-2)        /* valid request the library does not run (device, shape) */
#define INFLLMV2_WORKSPACE_TOO_SMALL (-3)
#define INFLLMV2_HIP_ERROR (-4)          /* a HIP runtime call or kernel launch failed */

typedef struct infllmv2_cfg {
  int32_t batch;            /* B >= 1 */
  int32_t n_q_heads;        /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;       /* Hkv >= 1; G = Hq / Hkv must divide 16 */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t block_size;       /* 64 */
  int32_t kernel_size;      /* 32 */
  int32_t kernel_stride;    /* 16 */
  int32_t top_k;            /* K >= 1 */
  int32_t dense_threshold;  /* rows with fewer visible keys attend densely; 0 = never */
  float softmax_scale;      /* <= 0 selects 1/sqrt(head_dim) */
} infllmv2_cfg;

/* Semantic kernels of the complete blocks j in [first_block, kv_len/64):
 * kernel m of block j = bf16(mean of k[b][g][64j+16m .. 64j+16m+31][:]), m = 0..2,
 * stored in the kbar layout above.
 * (QbitAI summary, "Model architecture: InfLLM v2", item 1: blocks are made of
 * fine-grained semantic kernels.) first_block lets a decode loop extend the
 * table when a block completes; blocks outside the range are not written. */
INFLLMV2_API int infllmv2_pool_kernels(const infllmv2_cfg* cfg, const void* k, int64_t kv_cap, int64_t kv_len,
                          int64_t first_block, void* kbar, void* stream);

/* Block scores of every query row (QbitAI summary, "Model architecture:
 * InfLLM v2", items 1 and 2): scores[b][g][i][j] = sum over the heads h of
 * group g of max over m of q[b][h][i] . (kernel m of block j), for j < floor(p_i/64);
 * -inf for every other j < nblk. Positions: p_i = q_pos0 + i, or q_pos0 for
 * every row when is_tree != 0 (all draft nodes score against the prefix). */
INFLLMV2_API int infllmv2_score_blocks(const infllmv2_cfg* cfg, const void* q, int32_t n_q, int64_t q_pos0,
                          int32_t is_tree, const void* kbar, int64_t kv_cap, float* scores,
                          void* stream);

/* Top-K blocks per (b, g, i) row (same summary and section: only the most
 * relevant blocks enter attention). With scores != NULL the rows are read from
 * a score tensor laid out as above; with scores == NULL the scores are computed
 * on the fly from q and kbar (the prefill path) and never stored. idx rows are
 * ascending, padded with -1. Positions as for infllmv2_score_blocks.
 * Candidate count floor(p/64) may be at most 4096. */
INFLLMV2_API int infllmv2_topk_blocks(const infllmv2_cfg* cfg, const float* scores, const void* q,
                         const void* kbar, int32_t n_q, int64_t q_pos0, int32_t is_tree,
                         int64_t kv_cap, int32_t* idx, void* stream);

/* Sparse causal attention for a chunk of n_q queries at positions
 * kv_len - n_q + i (a whole-sequence prefill has n_q == kv_len): each row
 * attends the 64 keys of each block in its group's idx row plus its own block
 * up to itself, or every visible key when it has fewer than dense_threshold of
 * them (QbitAI summary, "Model architecture: InfLLM v2": sparse attention over
 * the selected blocks in both prefill and decode, dense for short contexts). */
INFLLMV2_API int infllmv2_sparse_attn_prefill(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                 const void* k, const void* v, int64_t kv_cap, int64_t kv_len,
                                 const int32_t* idx, void* out, float* lse, void* stream);

/* Workspace (bytes, device memory) that infllmv2_sparse_attn_decode needs.
 * No initial contents are required; calls that share a workspace must not
 * overlap in time. */
INFLLMV2_API size_t infllmv2_decode_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q, int64_t kv_len);

/* Sparse attention of n_q new tokens against a KV cache, split across the
 * selected blocks and merged by log-sum-exp.
 *   tree_mask == NULL: rows sit at positions kv_len - n_q + i, as in prefill.
 *   tree_mask != NULL: draft-tree verification (QbitAI summary, section on
 *     fusing speculative sampling with long-context algorithms: the sparse
 *     kernel verifies tree drafts through a local mask kept as packed bits).
 *     Node i occupies cache slot P + i, P = kv_len - n_q, n_q <= 64; it attends
 *     its own selected blocks (chosen with is_tree = 1), the keys of block
 *     floor(P/64) before P, and every slot P + j whose bit j is set in
 *     tree_mask[b][i] (bit i must be set; bits j > i must be clear).
 * workspace: device memory of at least infllmv2_decode_workspace_bytes(). */
INFLLMV2_API int infllmv2_sparse_attn_decode(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                const void* k_cache, const void* v_cache, int64_t kv_cap,
                                int64_t kv_len, const int32_t* idx, const uint64_t* tree_mask,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/* A single-token decode step from block scores, in fewer launches (QbitAI
 * summary, "Model architecture: InfLLM v2", item 2: one block set per GQA
 * group, chosen by relevance): selects every group's top-K blocks from
 * scores [B][Hkv][1][nblk] (as written by infllmv2_score_blocks with n_q = 1,
 * q_pos0 = kv_len - 1), by the rule of infllmv2_topk_blocks, then attends
 * them exactly as infllmv2_sparse_attn_decode with n_q = 1 and no tree mask.
 * The selection runs inside the attention kernel (each split of a group
 * repeats it) instead of in a kernel of its own. Only entries j < (kv_len-1)/64
 * of a score row are candidates; the rest of the row may hold any value
 * (it is never chosen). Scores must not be NaN.
 *   idx_out: NULL, or [B][Hkv][1][K] int32 receiving the selected blocks.
 *   Requires top_k <= 64 and at most 4096 candidate blocks ((kv_len-1)/64),
 *   else INFLLMV2_UNSUPPORTED; workspace as for infllmv2_sparse_attn_decode
 *   with n_q = 1. */
INFLLMV2_API int infllmv2_sparse_attn_decode_scores(const infllmv2_cfg* cfg, const void* q,
                                       const void* k_cache, const void* v_cache, int64_t kv_cap,
                                       int64_t kv_len, const float* scores, int32_t* idx_out,
                                       void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* infllmv2_sparse_attn_decode_scores without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the split partials live in
 * a static device array of 16 MiB per GPU, allocated with the library's code
 * object and held until the process ends. This call allocates nothing and
 * calls no allocating routine. Same arguments, rules and results as
 * infllmv2_sparse_attn_decode_scores; a shape whose workspace
 * (infllmv2_decode_workspace_bytes with n_q = 1) exceeds 16 MiB returns
 * INFLLMV2_UNSUPPORTED. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (different streams or threads) race and
 * must be serialized by the caller. */
INFLLMV2_API int infllmv2_sparse_attn_decode_scores_noalloc(const infllmv2_cfg* cfg, const void* q,
                                               const void* k_cache, const void* v_cache,
                                               int64_t kv_cap, int64_t kv_len, const float* scores,
                                               int32_t* idx_out, void* out, float* lse,
                                               void* stream);

/* Bytes of workspace infllmv2_sparse_attn_prefill_backward needs for these
 * shapes (0 if the configuration is invalid). */
INFLLMV2_API size_t infllmv2_prefill_backward_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q,
                                                 int64_t kv_len);

/* Backward of infllmv2_sparse_attn_prefill: the gradients that make the
 * sparse attention trainable (QbitAI summary, "Model architecture: InfLLM
 * v2": native, trainable sparse attention; the block choice is a discrete
 * selection and passes no gradient). For upstream gradients dout of the
 * forward output out, with the forward's own key sets (idx, the own block up
 * to each row's position, dense rows below dense_threshold):
 *   dS_t = P_t (dout . v_t - dout . out),  P_t = exp(scale q.k_t - lse),
 *   dq = scale sum_t dS_t k_t,  dk_t = scale sum over rows dS_t q,
 *   dv_t = sum over rows P_t dout.
 *   q, out, dout [B][Hq][n_q][D] bf16; idx as for the forward; lse [B][Hq][n_q]
 *   fp32 as written by the forward (required);
 *   dq [B][Hq][n_q][D] fp32 (fully written); dk, dv [B][Hkv][kv_cap][D] fp32:
 *   rows < kv_len are written (zeros for keys no row attends), rows past
 *   kv_len are left untouched.
 *   The dk, dv sums of a key block attended by more than 4096 query rows
 *   (tokens x heads of the group) are split over workgroups and added with
 *   fp32 atomics, so their last bits may differ between runs; dk and dv must
 *   therefore be ordinary device memory (hipMalloc), not host or fine-grained
 *   memory. head_dim 64 runs the head_dim-128 kernels on copies zero-padded
 *   to 128 columns (zero columns change no dot product; the softmax scale
 *   stays the head_dim-64 one), kept in the workspace with the fp32 padded
 *   gradients. Workspace of at least
 *   infllmv2_prefill_backward_workspace_bytes(), no initial contents. */
INFLLMV2_API int infllmv2_sparse_attn_prefill_backward(const infllmv2_cfg* cfg, const void* q,
                                          int32_t n_q, const void* k, const void* v,
                                          int64_t kv_cap, int64_t kv_len, const int32_t* idx,
                                          const void* out, const float* lse, const void* dout,
                                          float* dq, float* dk, float* dv, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Dense attention of n_q queries at positions kv_len - n_q + i over the first
 * kv_len keys, causal (key <= position) or not: the short-context path
 * (QbitAI summary, "Model architecture: InfLLM v2": dense attention kept for
 * short sequences) and the reference the sparse path reduces to when K covers
 * every block. top_k and dense_threshold are ignored. */
INFLLMV2_API int infllmv2_dense_attn(const infllmv2_cfg* cfg, const void* q, int32_t n_q, const void* k,
                        const void* v, int64_t kv_cap, int64_t kv_len, int32_t causal, void* out,
                        float* lse, void* stream);

/* Bytes of workspace infllmv2_score_blocks_lse needs (0 if invalid). */
INFLLMV2_API size_t infllmv2_score_lse_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q,
                                          int64_t kv_cap);

/* LSE-normalized block scores for the top-K choice (QbitAI summary,
 * "Model architecture: InfLLM v2", item on more efficient operators: the
 * top-K blocks are picked with the help of a LogSumExp estimate; the pages
 * give no formula, so this is a reading). Per head h of a group, the kernel
 * scores s = softmax_scale * q_h . kbar[j][m] over every candidate kernel
 * (j < C, m < 3) are normalized by their log-sum-exp LSE_h, and
 *   scores[j] = sum over the group's heads of exp(max_m s_{h,j,m} - LSE_h)
 * for j < C, -inf otherwise (C as for infllmv2_score_blocks). Arguments,
 * layouts and row positions as infllmv2_score_blocks, plus a workspace of
 * infllmv2_score_lse_workspace_bytes() (per-head block values and per-tile
 * partial sums; no initial contents). The output feeds infllmv2_topk_blocks
 * (scores mode) and infllmv2_sparse_attn_decode_scores unchanged. */
INFLLMV2_API int infllmv2_score_blocks_lse(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                              int64_t q_pos0, int32_t is_tree, const void* kbar, int64_t kv_cap,
                              float* scores, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Decode-loop cache maintenance (QbitAI summary, efficiency evaluation: as
 * the context grows only the semantic-kernel representation grows with it, so
 * the kernel table is extended as blocks complete). Appends n_new tokens per
 * sequence: k_new, v_new [B][Hkv][n_new][D] bf16 go to rows len_b ..
 * len_b + n_new - 1 of k_cache, v_cache [B][Hkv][kv_cap][D], where len_b =
 * kv_lens[b] (device int64 [B], variable lengths; nullable) or kv_len (every
 * sequence; then kv_len + n_new <= kv_cap is checked). When kbar is given
 * (layout of infllmv2_pool_kernels), the kernels of every block the append
 * completes, blocks len_b/64 .. (len_b + n_new)/64 - 1, are pooled in the
 * same launch (from the cache rows before len_b and the appended rows of
 * k_new). Rows that would land at or past kv_cap are not written (device
 * lengths cannot be checked on the host). kv_lens is read, not updated: the
 * caller advances it. n_new = 0 is a no-op. An append touching more than
 * 2^31 - 1 (b, g, block) pairs returns INFLLMV2_UNSUPPORTED. */
INFLLMV2_API int infllmv2_append_kv(const infllmv2_cfg* cfg, const void* k_new, const void* v_new,
                       int32_t n_new, void* k_cache, void* v_cache, int64_t kv_cap,
                       const int64_t* kv_lens, int64_t kv_len, void* kbar, void* stream);

/* Block scores of one new token per sequence in a batch of variable lengths
 * (the scoring of infllmv2_score_blocks): sequence b's token sits at position
 * kv_lens[b] - 1 (device int64 [B], each >= 1), so its candidates are the
 * complete blocks j < (kv_lens[b] - 1)/64. q [B][Hq][1][D]; scores
 * [B][Hkv][1][nblk] fp32 with nblk = ceil(kv_cap / 64), -inf past each
 * sequence's candidates. */
INFLLMV2_API int infllmv2_score_blocks_varlen(const infllmv2_cfg* cfg, const void* q,
                                 const int64_t* kv_lens, const void* kbar, int64_t kv_cap,
                                 float* scores, void* stream);

/* Bytes of workspace infllmv2_sparse_attn_decode_varlen needs when no
 * sequence is longer than kv_len_max (0 if the configuration is invalid). */
INFLLMV2_API size_t infllmv2_decode_varlen_workspace_bytes(const infllmv2_cfg* cfg,
                                              int64_t kv_len_max);

/* infllmv2_sparse_attn_decode_scores for a batch of variable lengths: one new
 * token per sequence at position kv_lens[b] - 1 (device int64 [B]), with
 * 1 <= kv_lens[b] <= kv_len_max <= kv_cap (values outside are clamped to that
 * range on the device); selection from scores (as written by
 * infllmv2_score_blocks_varlen), the own block and the dense switch apply per
 * sequence. Workspace: infllmv2_decode_varlen_workspace_bytes(kv_len_max). */
INFLLMV2_API int infllmv2_sparse_attn_decode_varlen(const infllmv2_cfg* cfg, const void* q,
                                       const void* k_cache, const void* v_cache, int64_t kv_cap,
                                       const int64_t* kv_lens, int64_t kv_len_max,
                                       const float* scores, int32_t* idx_out, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Sliding-window causal attention: query i at position p = kv_len - n_q + i
 * attends keys max(0, p - window + 1) .. p (QbitAI summary, section on fusing
 * speculative sampling, quantization and long-context algorithms: the draft
 * model uses sliding-window attention while the target model uses the sparse
 * kernels). Serves both a draft prefill (n_q = prompt length) and its decode
 * steps (n_q = 1 with the new token's K/V already in the cache). Layouts as
 * infllmv2_dense_attn; top_k and dense_threshold are ignored; window >= 1
 * (values above kv_len act as kv_len, i.e. dense causal). head_dim 64 or
 * 128. */
INFLLMV2_API int infllmv2_sliding_window_attn(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                 const void* k, const void* v, int64_t kv_cap, int64_t kv_len,
                                 int64_t window, void* out, float* lse, void* stream);

/* Static text for a status code. */
INFLLMV2_API const char* infllmv2_strerror(int status);

/* Message describing the last failed call on this thread ("" if none). */
INFLLMV2_API const char* infllmv2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* INFLLMV2_H */
