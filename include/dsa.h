/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-Sparse-Attention path used by
 * GLM-5.3-Flash: kpool indexer (pools, scores, top-k, expansion) and sparse
 * NoPE MLA over an INT8 latent cache.
 *
 * Page citations use these short names:
 *   [Flash]   "GLM-5.3-Flash" (pypto-lib model staging page)
 *   [Kernels] "GLM-5.3 Kernels" (store_int8 / sparse MLA kernel release)
 *   [Ref]     "Module glm5next_dsa_ref" (DSA + kpool indexer CPU reference docs)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers documented as "device" point to GPU memory on the device that is
 *    current for the calling thread; "host" pointers are read before the call
 *    returns.  The caller owns every buffer, including workspaces; the library
 *    allocates nothing and keeps no per-call state (it caches device
 *    properties only; dsa_time_next_scoring_launch keeps two event handles
 *    per thread until the next scoring launch) and is safe to call from
 *    several host threads.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream), never synchronises, and returns a dsa_status.  Only host-visible
 *    arguments are validated; on any error nothing is launched.  Device data
 *    (slots, indices, positions, lengths) is trusted: out-of-range positive
 *    indices and duplicate slots are outside the contract, as for the pages'
 *    low-level API ([Kernels] Install: contract paragraph).
 *  - Outputs are written, never read-modify-written, and every entry of every
 *    output is written, so uninitialised destinations are safe ([Ref] Traps:
 *    the sentinel and the fully written destination).
 *  - bf16 buffers hold raw bf16 bit patterns (uint16_t).
 *  - Position x of sequence b (0 <= x < its length) lives at cache row
 *    row_base[b] + x and at indexer-state row tok_base[b] + x; positions below
 *    first_valid[b] are left padding.  Pool p of sequence b lives at pool row
 *    pool_base[b] + p and covers positions first_valid[b] + kpool*p + s,
 *    s in [0, kpool) ([Ref] Traps: pools start at the first valid token).
 *  - A query at position q_pos of sequence b sees positions first_valid[b]..
 *    q_pos (itself included) and the n_vis = (q_pos - first_valid + 1) / kpool
 *    pools whose slots all lie in that range (0 when q_pos < first_valid)
 *    ([Ref] Functions: visible; Traps: a pool needs all of its slots).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL = -1,        /* a required pointer is NULL */
    DSA_ERR_DIMS = -2,        /* inconsistent or non-positive dims */
    DSA_ERR_DTYPE = -3,       /* dtype code not accepted by this call */
    DSA_ERR_ALIGN = -4,       /* pointer or leading dimension misaligned */
    DSA_ERR_WIDTH = -5,       /* out_width < index_topk + kpool - 1 */
    DSA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
    DSA_ERR_UNSUPPORTED = -7, /* valid dims this build has no kernel for */
    DSA_ERR_HIP = -8,         /* a HIP runtime call or launch failed */
    DSA_ERR_SIZE = -9,        /* negative count or a stride smaller than needed */
    DSA_ERR_TIMEOUT = -10,    /* dsa_decode_step_status: a wait inside the launch timed out */
    DSA_ERR_SCRATCH = -11     /* dsa_sparse_mla_noalloc: the call needs more than its fixed scratch */
} dsa_status;

typedef enum dsa_dtype {
    DSA_F32 = 0,
    DSA_BF16 = 1
} dsa_dtype;

/*
 * Indexer + MLA geometry, read from the model config and never defaulted
 * ([Ref] Structs: DsaDims).  GLM-5.3-Flash: idx_heads 32, idx_dim 128,
 * kpool 4, index_topk 2048 ([Flash] checkpoint table), out_width 2176,
 * latent_dim 512, row_bytes 528, mla_heads 16 per rank ([Kernels] Included).
 * Required: all positive; index_topk % kpool == 0 (select_k = index_topk /
 * kpool pools); out_width >= index_topk + kpool - 1; row_bytes ==
 * round_up(latent_dim + 4, 16); ln_eps >= 0.
 */
typedef struct dsa_dims {
    int32_t idx_heads;
    int32_t idx_dim;
    int32_t kpool;
    int32_t index_topk;
    int32_t out_width;
    int32_t mla_heads;
    int32_t latent_dim;
    int32_t row_bytes;
    float ln_eps;
} dsa_dims;

/* Per-sequence layout; every pointer is a device array of num_seqs entries. */
typedef struct dsa_seqs {
    const int32_t* first_valid;  /* left-padding length f_b (first valid position) */
    const int64_t* row_base;     /* cache row of position 0 */
    const int64_t* tok_base;     /* indexer-state (k, gate) row of position 0 */
    const int64_t* pool_base;    /* pool row of pool 0 */
} dsa_seqs;

/*
 * Paged caches -- [Kernels] Install (the INT8 cache allocated as [n / 256,
 * 256, 528]: blocks of 256 rows) and [Flash] What already exists (slot
 * mappings for the latent, the per-token indexer state and the pooled state).
 * A sequence's block table maps its i-th block of 256 positions to a physical
 * block id k; block k holds latent cache rows 256 k .. 256 k + 255, indexer
 * state (k, gate) rows 256 k .. 256 k + 255 and pool rows 64 k .. 64 k + 63.
 * Position x of sequence b is row 256 * block_table[b * table_stride + x / 256]
 * + x % 256; pool p is row 64 * block_table[b * table_stride + p / 64] + p % 64.
 * The table must cover every position and pool a call touches.  New INT8 rows
 * are written with dsa_store_int8 at their physical slots (the slot mapping);
 * dsa_sparse_mla takes the index list the paged selection writes, whose
 * entries are physical rows.
 */
typedef struct dsa_paged_seqs {
    const int32_t* first_valid;  /* device [num_seqs]: left-padding length */
    const int32_t* block_table;  /* device [num_seqs, table_stride]: physical block ids */
    int32_t table_stride;        /* host: entries per sequence in block_table */
} dsa_paged_seqs;

int dsa_abi_version(void);
const char* dsa_status_string(int status);

/*
 * store_int8 -- [Kernels] Included: each latent row becomes one INT8 row of
 * row_bytes bytes: latent_dim int8 codes, then the fp32 scale (little endian),
 * then zero bytes up to row_bytes (512 + 4 + 12 = 528).  Per row:
 *   amax = max|x|, s = fp32(max(amax, 1e-4) / 127) (IEEE division),
 *   code = clamp(round_half_even(fp32(x / s)), -127, 127).
 *   latent  device, [n, ld] of latent_dtype (DSA_BF16 or DSA_F32), rows of
 *           latent_dim contiguous values; 16-byte aligned base and row pitch.
 *   slots   device int64 [n]: destination cache row of each latent row;
 *           negative = skip (padding).  Must be < cache_rows and distinct.
 *   cache   device, [cache_rows, row_bytes] bytes, 16-byte aligned.
 */
int dsa_store_int8(const dsa_dims* dims, const void* latent, int latent_dtype,
                   int64_t n, int64_t ld, const int64_t* slots,
                   int8_t* cache, int64_t cache_rows, void* stream);

/*
 * index_pools -- [Ref] Traps and Functions (layer_norm, pool_states): for
 * every pool p in [pool_begin[b], pool_end[b]) of every sequence b,
 *   y_s = LayerNorm(k[t_s]) * ln_w + ln_b   (mean-subtracted, biased variance, ln_eps)
 *   a_s[c] = softmax over the kpool slots s of gate[t_s][c]   (per channel)
 *   pool[p][c] = sum_s a_s[c] * y_s[c], stored as bf16 (round to nearest even)
 * with t_s = tok_base[b] + first_valid[b] + kpool*p + s.
 *   k, gate     device [tokens, idx_dim] of kg_dtype (DSA_BF16 or DSA_F32)
 *   ln_w, ln_b  device fp32 [idx_dim]
 *   pool_begin, pool_end  device int32 [num_seqs]; the caller guarantees that
 *               all kpool tokens of every listed pool exist.
 *   max_pools   host: >= max_b (pool_end[b] - pool_begin[b]) (sizes the grid)
 *   pools       device bf16 [*, idx_dim]
 * Supported: kpool 4, idx_dim in {32, 128}.
 */
int dsa_index_pools(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype,
                    const float* ln_w, const float* ln_b, const dsa_seqs* seqs,
                    int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                    int32_t max_pools, uint16_t* pools, void* stream);

/*
 * append_tokens -- a step's new tokens in one launch: exactly dsa_store_int8
 * (latent, n, ld, slots, cache, cache_rows) followed by dsa_index_pools (k,
 * gate, ln_w, ln_b, seqs, num_seqs, pool_begin, pool_end, max_pools, pools),
 * with one dtype (DSA_BF16 or DSA_F32) for latent, k and gate.  The results
 * are bit-identical to the two calls.  The two parts touch disjoint buffers:
 * the pools are built from k and gate, not from the cache rows.
 *   n == 0 skips the rows (latent, slots, cache may be NULL); max_pools == 0
 *   skips the pools (k .. pools and seqs may be NULL).
 * Supported: the union of the two calls' limits (latent_dim in {64, 128,
 * 256, 512}; kpool 4, idx_dim in {32, 128}).
 */
int dsa_append_tokens(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                      const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                      const void* gate, const float* ln_w, const float* ln_b, const dsa_seqs* seqs,
                      int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                      int32_t max_pools, uint16_t* pools, void* stream);

/*
 * index_scores -- [Ref] Functions (index_scores): matmul, ReLU, head-weighted
 * sum.  For query t (sequence q_seq[t], position q_pos[t]) and pool p:
 *   scores[t][p] = sum_h w[t][h] * max(0, q_idx[t][h] . pool[p])   for p < n_vis(t)
 *   scores[t][p] = -inf                                            for n_vis(t) <= p < score_stride
 * bf16 products, fp32 accumulation.
 *   q_idx   device bf16 [T, idx_heads, idx_dim]; w device fp32 [T, idx_heads]
 *   pools   device bf16; rows pool_base[b] + p must hold built pools for every
 *           p < n_vis(t) of every query t of sequence b
 *   q_seq, q_pos  device int32 [T]
 *   scores  device fp32 [T, score_stride]; score_stride must be >= every
 *           query's n_vis.
 * Uses the MFMA kernel for idx_heads 32 x idx_dim 128, a vector kernel otherwise.
 */
int dsa_index_scores(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                     const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                     const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                     int32_t score_stride, float* scores, void* stream);

/*
 * topk_select -- [Ref] Functions (topk_pools); [Flash] Stream C
 * (indexer_topk512): select K = min(select_k, n_vis(t)) pools per query by
 * (score descending, pool id ascending; -0 equals +0), and write their ids
 * in ascending order to pool_ids[t][0..K), then -1 up to select_k.  When
 * n_vis <= select_k every visible pool is selected.  NaN scores are outside
 * the contract.  Supported: kpool 4, select_k <= 1024 and score_stride <=
 * 262,144 pools.
 *   scores    device fp32 [T, score_stride] (as written by dsa_index_scores)
 *   pool_ids  device int32 [T, select_k]
 *   workspace device scratch, >= dsa_topk_workspace_bytes(dims, T,
 *             score_stride) bytes, 256-byte aligned; needs no initialisation
 *             and holds nothing between calls.  Calls sharing one workspace
 *             must not overlap.  Rows of at most 40,960 pools are selected
 *             in one pass and need none (the size is then 0 and workspace
 *             may be NULL).
 */
size_t dsa_topk_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride);
int dsa_topk_select(const dsa_dims* dims, const float* scores, int32_t score_stride,
                    const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                    const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * topk_select_expand -- topk_select and expand_selection in one launch: the
 * same selection as dsa_topk_select, written as the expanded index list
 * (exactly what dsa_expand_selection would produce from it) and, when
 * pool_ids is not NULL, also as pool ids.  Same workspace contract.
 *   pool_ids  device int32 [T, select_k] or NULL
 *   indices   device int32 [T, out_width]
 */
int dsa_topk_select_expand(const dsa_dims* dims, const float* scores, int32_t score_stride,
                           const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * index_scores_select -- dsa_index_scores followed by dsa_topk_select_expand,
 * with the same results (scores, pool_ids, indices), in two launches: for
 * decode batches (T <= 64, 32 x 128 indexer heads, select_k <= 512,
 * score_stride <= 65,536) the scoring pass also keeps each 64-pool group's
 * best pools, so the selection reads those lists instead of a per-tile pass
 * over the scores; other shapes run the two calls unchanged.
 *   arguments as dsa_index_scores and dsa_topk_select_expand
 *   workspace  device, >= dsa_index_scores_select_workspace_bytes(dims, T,
 *              score_stride) bytes, 256-byte aligned; scratch only.
 */
size_t dsa_index_scores_select_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride);
/*
 * The two halves of dsa_index_scores_select for decode shapes, as separate
 * calls sharing one workspace (same size): dsa_index_scores_groups writes the
 * scores and, into the workspace, each 64-pool group's best pools;
 * dsa_topk_select_groups then selects from those lists (reading the scores
 * only if it must fall back to an exact pass).  Other shapes:
 * DSA_ERR_UNSUPPORTED.
 */
int dsa_index_scores_groups(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                            const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                            const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                            int32_t score_stride, float* scores, void* workspace,
                            size_t workspace_bytes, void* stream);
int dsa_topk_select_groups(const dsa_dims* dims, const float* scores, int32_t score_stride,
                           const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * append_scores_groups -- dsa_append_tokens followed by
 * dsa_index_scores_groups, with the same results (cache rows, pools, scores
 * and the group lists in the workspace), in one launch when the new tokens
 * are bf16 and idx_dim is 128 (else the two launches).  The scoring part of
 * the launch runs while the new rows and pools are still being written: a
 * wave whose 64-pool group holds a pool the step completes builds that pool
 * itself (the same arithmetic as dsa_index_pools, so the same bits) and
 * scores it from registers, never from the pools buffer.
 *   dtype .. pools      as dsa_append_tokens (seqs and num_seqs shared)
 *   q_idx .. workspace  as dsa_index_scores_groups; pools is the buffer both
 *                       parts use
 *   T == 0 or score_stride == 0 does the new tokens only.
 * Supported: what both calls support; DSA_ERR_UNSUPPORTED otherwise.
 */
int dsa_append_scores_groups(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                             const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                             const void* gate, const float* ln_w, const float* ln_b,
                             const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                             uint16_t* pools, const uint16_t* q_idx, const float* w, const dsa_seqs* seqs,
                             int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                             int32_t score_stride, float* scores, void* workspace, size_t workspace_bytes,
                             void* stream);
/*
 * time_next_scoring_launch -- measurement hook.  The next scoring launch
 * made on the calling thread for 32 x 128 indexer heads (by
 * dsa_append_scores_groups, dsa_index_scores_groups, dsa_index_scores_select,
 * dsa_index_scores, dsa_index_select_chunked or their INT8-pool forms)
 * records start_event
 * when the kernel starts and stop_event when it ends (hipExtLaunchKernel),
 * so that hipEventElapsedTime gives the kernel's own duration, without the
 * gap between launches.  One-shot; both NULL cancels.  The events are HIP
 * events created beforehand on the launch's device; the library does not
 * own them.  Returns DSA_ERR_NULL if exactly one of them is NULL.
 */
int dsa_time_next_scoring_launch(void* start_event, void* stop_event);
int dsa_index_scores_select(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                            const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                            const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                            int32_t score_stride, float* scores, int32_t* pool_ids, int32_t* indices,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * index_pools_paged / index_scores_groups_paged / topk_select_groups_paged --
 * dsa_index_pools, dsa_index_scores_groups and dsa_topk_select_groups over
 * paged caches: the same pools, scores, group lists and selection, bit for
 * bit, with every k / gate row, pool row and index-list entry taken through
 * the block table.  Arguments as the flat calls, with dsa_paged_seqs in place
 * of dsa_seqs; the scoring workspace is the flat one
 * (dsa_index_scores_select_workspace_bytes).  Supported: what the flat calls
 * support.
 */
int dsa_index_pools_paged(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype,
                          const float* ln_w, const float* ln_b, const dsa_paged_seqs* seqs, int32_t num_seqs,
                          const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                          uint16_t* pools, void* stream);
int dsa_index_scores_groups_paged(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                                  const uint16_t* pools, const dsa_paged_seqs* seqs, int32_t num_seqs,
                                  const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                                  float* scores, void* workspace, size_t workspace_bytes, void* stream);
int dsa_topk_select_groups_paged(const dsa_dims* dims, const float* scores, int32_t score_stride,
                                 const dsa_paged_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * INT8 pool cache -- [Flash] What is quantized (the indexer state cache row:
 * the sibling port stores its indexer cache as INT8 with one FP32 scale per
 * row).  A pool is kept as idx_dim INT8 codes (one row of idx_dim bytes) and
 * one fp32 scale, 132 bytes per pool instead of 256 in bf16.  The codes and
 * the scale are those of dsa_store_int8's quantiser applied to the pool's
 * fp32 state (amax over the row floored at 1e-4, s = amax / 127 in IEEE
 * fp32, round half to even, +-127); there is no bf16 step in between.
 * Scores are computed on the dequantised pools:
 *   scores[t][p] = sum_h w[t][h] * max(0, q_idx[t][h] . (scale[p] * code[p]))
 * (as s * sum_h w[h] * relu(q . code), bf16 products and fp32 sums), -inf
 * past the visible pools, exactly as dsa_index_scores lays them out.
 *
 * index_pools_int8 -- dsa_index_pools in the INT8 form.
 *   k .. max_pools  as dsa_index_pools
 *   pool_codes   device int8 [*, idx_dim], row pool_base[b] + p; 16-byte aligned
 *   pool_scales  device fp32 [*], same rows
 *   pools_f32    device fp32 [*, idx_dim] or NULL: when set, also receives
 *                each pool's fp32 values before quantisation (for checks)
 * Supported: kpool 4, idx_dim in {32, 128}.
 */
int dsa_index_pools_int8(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype,
                         const float* ln_w, const float* ln_b, const dsa_seqs* seqs, int32_t num_seqs,
                         const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                         int8_t* pool_codes, float* pool_scales, float* pools_f32, void* stream);
/*
 * index_scores_int8 / index_scores_groups_int8 / append_scores_groups_int8 --
 * dsa_index_scores, dsa_index_scores_groups and dsa_append_scores_groups over
 * INT8 pools (pool_codes, pool_scales in place of the bf16 pools; the new
 * tokens' pools are built in the INT8 form).  The group lists in the
 * workspace are those the selection calls read (dsa_topk_select_groups,
 * dsa_topk_sparse_mla), with the same workspace size.  In the single launch,
 * a pool the step completes is built, quantised and scored by the wave that
 * scores its group, so its score is the one a separate scoring pass over the
 * stored pool gives.
 * Supported: idx_heads 32, idx_dim 128, kpool 4, T <= 64; bf16 new tokens
 * for the single launch; else DSA_ERR_UNSUPPORTED.
 */
int dsa_index_scores_int8(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                          const int8_t* pool_codes, const float* pool_scales, const dsa_seqs* seqs,
                          int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                          int32_t score_stride, float* scores, void* stream);
int dsa_index_scores_groups_int8(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                                 const int8_t* pool_codes, const float* pool_scales, const dsa_seqs* seqs,
                                 int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                 int32_t score_stride, float* scores, void* workspace, size_t workspace_bytes,
                                 void* stream);
int dsa_append_scores_groups_int8(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                                  const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                                  const void* gate, const float* ln_w, const float* ln_b,
                                  const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                  int8_t* pool_codes, float* pool_scales, const uint16_t* q_idx, const float* w,
                                  const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                                  const int32_t* q_pos, int32_t T, int32_t score_stride, float* scores,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * append_scores_groups_shared -- dsa_append_scores_groups (pool_scales NULL:
 * bf16 pools) or dsa_append_scores_groups_int8 (pool_scales set: `pools`
 * holds the INT8 code rows) for batches whose queries come in runs of one
 * sequence, as in a speculative decode step that scores the accepted token
 * and its drafts together ([Flash] Deployment target: MTP with 3 speculative
 * tokens; Stream C: indexer_share_mtp).  Consecutive queries with the same
 * q_seq form runs of at most `share` (1 .. 4); the pools of a run's sequence
 * are read once for the whole run instead of once per query.  Results
 * (cache rows, pools, scores, group lists) are bit for bit those of the
 * one-query call; share == 1 is that call.  Arguments as
 * dsa_append_scores_groups, plus pool_scales and share; n == 0 and
 * max_pools == 0 score only.
 * Supported: what dsa_append_scores_groups_int8 supports (bf16 new tokens).
 */
int dsa_append_scores_groups_shared(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                                    const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                                    const void* gate, const float* ln_w, const float* ln_b,
                                    const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                    void* pools, float* pool_scales, const uint16_t* q_idx, const float* w,
                                    const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t T, int32_t score_stride, float* scores,
                                    void* workspace, size_t workspace_bytes, int32_t share, void* stream);

/*
 * index_select_chunked -- index_scores and topk_select_expand for many
 * queries (a prefill chunk) with a bounded scoring workspace: the queries are
 * taken `chunk` at a time, each group's fp32 scores [chunk, score_stride] are
 * written to the workspace, selected and expanded, then overwritten by the
 * next group (the pages' integration keeps the indexer's workspaces bounded:
 * [Kernels] Included).  pool_ids and indices are those dsa_index_scores +
 * dsa_topk_select_expand give for all T queries at once; the scores are not
 * kept.  Rows of at most 40,960 pools are selected in one pass over their
 * scores.  Past that, for 32 x 128 indexer heads, select_k <= 512 and
 * score_stride <= 65,536 the scoring pass also keeps each 64-pool group's
 * best pools and the selection reads those lists (as
 * dsa_index_scores_select does for decode); other geometries sort 256-pool
 * tiles of the scores.
 *   q_idx .. score_stride   as dsa_index_scores
 *   chunk      host: queries per group (1 .. 65,535); the workspace holds
 *              chunk x score_stride scores, e.g. 512 x 33,792 x 4 B = 69 MB
 *   pool_ids   device int32 [T, select_k] or NULL; indices device int32
 *              [T, out_width]
 *   workspace  device, >= dsa_index_select_chunked_workspace_bytes(dims,
 *              chunk, score_stride) bytes, 256-byte aligned; scratch only.
 * Supported: what dsa_topk_select supports.
 */
size_t dsa_index_select_chunked_workspace_bytes(const dsa_dims* dims, int32_t chunk, int32_t score_stride);
int dsa_index_select_chunked(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                             const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                             const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                             int32_t chunk, int32_t* pool_ids, int32_t* indices, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * expand_selection -- [Ref] Functions (expand_selection) and Traps (the -1
 * sentinel, fully written output): for each query, the selected pools (the
 * leading non-negative entries of pool_ids[t], ascending) become their kpool
 * cache rows row_base + first_valid + kpool*p + s, then the visible tail
 * positions first_valid + kpool*n_vis .. q_pos follow (at most kpool - 1),
 * then -1 fills the row up to out_width.
 *   pool_ids  device int32 [T, select_k], front-packed
 *   indices   device int32 [T, out_width]
 */
int dsa_expand_selection(const dsa_dims* dims, const int32_t* pool_ids, const dsa_seqs* seqs,
                         int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                         int32_t T, int32_t* indices, void* stream);

/*
 * sparse_mla -- [Kernels] Included and Install (triton_mla_sparse_attention:
 * fused INT8 dequant, one shared K/V latent, split-KV decode, bf16 products,
 * fp32 softmax); [Ref] Functions (mla_masked_attention).  For query t, head h:
 *   J = { j : indices[t][j] >= 0 },  K_j = V_j = code_j * scale_j (the stored row)
 *   z_j = scale * q[t][h] . K_j,  out[t][h] = sum_j softmax_j(z) V_j,
 *   lse[t][h] = log(sum_j exp(z_j)) (natural log).
 * Negative entries are skipped wherever they sit; an empty J gives out = 0
 * and lse = -inf.  Bitwise run-to-run deterministic for a fixed num_splits.
 *   q        device [T, mla_heads, latent_dim] of q_dtype (DSA_BF16 or DSA_F32)
 *   cache    device [cache_rows, row_bytes] (rows written by dsa_store_int8)
 *   indices  device int32 [T, out_width]; valid entries < cache_rows
 *   out      device [T, mla_heads, latent_dim] of out_dtype (DSA_F32 or DSA_BF16)
 *   lse      device fp32 [T, mla_heads] or NULL
 *   num_splits  0 = choose from T, heads and the device's CU count; otherwise
 *            the number of list partitions per query (clamped to what the
 *            list width allows).
 *   workspace device, >= dsa_sparse_mla_workspace_bytes(dims, T, num_splits)
 *            bytes, 256-byte aligned (NULL allowed when that size is 0).
 * bf16 q with latent_dim 512 and mla_heads % 16 == 0 runs on MFMA; other
 * shapes and fp32 q use an fp32 vector kernel.
 */
size_t dsa_sparse_mla_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t num_splits);
int dsa_sparse_mla(const dsa_dims* dims, const void* q, int q_dtype, const int8_t* cache,
                   int64_t cache_rows, const int32_t* indices, int32_t T, float scale,
                   void* out, int out_dtype, float* lse, int32_t num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_mla_noalloc -- dsa_sparse_mla for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same results bit for bit (for the same num_splits).  The
 * split partials go to a fixed device array of
 * dsa_sparse_mla_noalloc_scratch_bytes() bytes (16 MiB) that the library
 * holds on each device it runs on until the process ends; its address is
 * resolved on the first call on a device.  The call allocates nothing.
 * A call whose partials would not fit (dsa_sparse_mla_workspace_bytes(dims,
 * T, num_splits) larger than that) returns DSA_ERR_SCRATCH and launches
 * nothing.  All calls on one GPU share that GPU's array: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  The array needs no initialisation.
 */
size_t dsa_sparse_mla_noalloc_scratch_bytes(void);
int dsa_sparse_mla_noalloc(const dsa_dims* dims, const void* q, int q_dtype, const int8_t* cache,
                           int64_t cache_rows, const int32_t* indices, int32_t T, float scale,
                           void* out, int out_dtype, float* lse, int32_t num_splits, void* stream);

/*
 * topk_sparse_mla -- dsa_topk_select_groups followed by dsa_sparse_mla over
 * the list it writes, with the same results bit for bit (pool_ids, indices,
 * out, lse for the same num_splits), in two launches instead of three: each
 * attention workgroup makes its query's selection from the group lists
 * itself ([Ref] Functions: topk_pools, expand_selection,
 * mla_masked_attention) and reads its rows from the ids it holds; the
 * partials are then merged as in dsa_sparse_mla.
 *   dims .. T, pool_ids, indices   as dsa_topk_select_groups (pool_ids may
 *                  be NULL; indices is written in full)
 *   select_workspace, select_workspace_bytes   the group lists, as written
 *                  by dsa_index_scores_groups / dsa_append_scores_groups for
 *                  the same queries
 *   q .. num_splits   as dsa_sparse_mla
 *   mla_workspace  device, >= dsa_sparse_mla_workspace_bytes(dims, T,
 *                  num_splits) bytes, 256-byte aligned (NULL allowed when
 *                  that size is 0).
 * Supported: what dsa_topk_select_groups supports, with score_stride > 0;
 * else DSA_ERR_UNSUPPORTED.  Attention shapes the one-launch form does not
 * cover (not bf16 q, latent_dim != 512, or more than one 16-head tile per
 * workgroup) run the two calls.
 */
int dsa_topk_sparse_mla(const dsa_dims* dims, const float* scores, int32_t score_stride,
                        const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                        const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                        const void* select_workspace, size_t select_workspace_bytes, const void* q,
                        int q_dtype, const int8_t* cache, int64_t cache_rows, float scale, void* out,
                        int out_dtype, float* lse, int32_t num_splits, void* mla_workspace,
                        size_t mla_workspace_bytes, void* stream);

/*
 * decode_step -- one launch for a decode step's index_scores, topk_select,
 * expand_selection and sparse_mla (the chain of [Ref] Functions:
 * index_scores, topk_pools, expand_selection, mla_masked_attention, and
 * [Kernels] Included: split-KV decode with a combine).  The results are the
 * ones the separate calls produce: the list dsa_topk_select_expand would
 * write (same selection, same tie rule) as indices and pool_ids when not
 * NULL, bit for bit, and out/lse as dsa_sparse_mla over that list up to the
 * grouping of its floating-point sums (a few fp32 ulps).
 * The step's new tokens must already be stored (dsa_store_int8) and the
 * pools they complete built (dsa_index_pools).
 *   q_idx, w, pools, seqs, q_seq, q_pos   as dsa_index_scores
 *   score_stride   >= every query's visible pool count; <= 65,536
 *   q, cache, scale, out, out_dtype, lse  as dsa_sparse_mla (q bf16 only)
 *   pool_ids       device int32 [T, select_k] or NULL
 *   indices        device int32 [T, out_width] or NULL
 *   workspace      device, >= dsa_decode_step_workspace_bytes(dims, T,
 *                  score_stride) bytes, 256-byte aligned.  It must be
 *                  zero-filled before its first use; every call leaves its
 *                  control words zero again, so one allocation serves any
 *                  number of calls.  Calls sharing a workspace must not
 *                  overlap.  The uint32 at byte offset 8 of the workspace
 *                  becomes nonzero if a wait inside the launch ever timed out
 *                  (the results of that call are then invalid).
 * Supported: idx_heads 32, idx_dim 128, kpool 4, select_k <= 512,
 * latent_dim 512, mla_heads a multiple of 16 up to 64, T <= 64,
 * out_width <= 8192; else DSA_ERR_UNSUPPORTED.
 */
size_t dsa_decode_step_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride);
/*
 * decode_step_status -- reads the error word of a dsa_decode_step workspace
 * after the work enqueued on `stream` so far (this call synchronises the
 * stream): DSA_OK, or DSA_ERR_TIMEOUT when a wait inside some launch that
 * used the workspace timed out (that launch's outputs are then invalid; the
 * word stays set until the caller zero-fills the workspace again).
 *   workspace  device, as passed to dsa_decode_step; workspace_bytes >= 12.
 */
int dsa_decode_step_status(const void* workspace, size_t workspace_bytes, void* stream);
int dsa_decode_step(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                    const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                    const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                    const void* q, int q_dtype, const int8_t* cache, int64_t cache_rows,
                    float scale, void* out, int out_dtype, float* lse, int32_t* pool_ids,
                    int32_t* indices, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
