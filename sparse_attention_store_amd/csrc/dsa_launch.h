// Internal launchers: each validates nothing (dsa_api.cpp does) and enqueues
// its kernels on the given stream.  They return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa_host {

hipError_t launch_store_int8(const dsa_dims& d, const void* latent, int dtype, int64_t n,
                             int64_t ld, const int64_t* slots, int8_t* cache, hipStream_t s);

hipError_t launch_index_pools(const dsa_dims& d, const void* k, const void* gate, int dtype,
                              const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                              int32_t num_seqs, const int32_t* pool_begin,
                              const int32_t* pool_end, int32_t max_pools, uint16_t* pools,
                              hipStream_t s);
hipError_t launch_append_tokens(const dsa_dims& d, int dtype, const void* latent, int64_t n, int64_t ld,
                                const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                uint16_t* pools, hipStream_t s);

hipError_t launch_index_scores(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                               const uint16_t* pools, const dsa_seqs& seqs, int32_t num_seqs,
                               const int32_t* q_seq,
                               const int32_t* q_pos, int32_t T, int32_t stride, float* scores,
                               hipStream_t s);

// Group lists for at most 64 queries of rows up to 262,144 pools (64-pool
// groups up to 65,536 pools, 256-pool groups past that): the flat decode
// scoring launches and the selections from their lists.
bool scores_select_grouped(const dsa_dims& d, int32_t T, int32_t stride);
// The same up to 65,536 pools (64-pool groups only): the paged and shared-run
// scoring kernels and the prefill kernel's lists.
bool scores_lists_short(const dsa_dims& d, int32_t T, int32_t stride);
// Scores plus each 64-pool group's best pools, for any T (group-list geometry:
// scores_lists_short(d, min(T, 64), stride)); the lists are laid out as
// launch_scores_with_groups lays them out for T queries.
hipError_t launch_scores_lists(const dsa_dims& d, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                               const dsa_seqs& seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                               int32_t T, int32_t stride, float* scores, void* ws, hipStream_t s);
size_t scores_select_group_bytes(int32_t T);
hipError_t launch_scores_with_groups(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                     const uint16_t* pools, const dsa_seqs& seqs, int32_t num_seqs,
                                     const int32_t* q_seq,
                                     const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                     hipStream_t s);
bool append_scores_fused(const dsa_dims& d, int dtype);
// Events the next scoring launch of launch_append_scores_groups on this
// thread records around the kernel (one-shot).
void time_next_scoring_launch(hipEvent_t start, hipEvent_t stop);
hipError_t launch_append_scores_groups(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                       const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                       const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                       const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                       uint16_t* pools, const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                       const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                       hipStream_t s);
hipError_t launch_topk_groups(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                              const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                              int32_t* indices, const void* ws, hipStream_t s);

// k_scores_runs: runs of up to `share` consecutive queries of one sequence
// share one pass over its pools; pools are bf16 rows, or INT8 code rows when
// scales is not null.  n == 0 and max_pools == 0: no new tokens.
hipError_t launch_append_scores_groups_runs(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                            const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                            const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                                            int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                                            int32_t max_pools, void* pools, float* scales, const uint16_t* q_idx,
                                            const float* w, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                            int32_t stride, float* scores, void* ws, int share, hipStream_t s);

// Paged caches (paged.h): every position / pool row through a block table.
hipError_t launch_index_pools_paged(const dsa_dims& d, const void* k, const void* gate, int dtype, const float* ln_w,
                                    const float* ln_b, const int32_t* first_valid, const int32_t* table,
                                    int32_t table_stride, int32_t num_seqs, const int32_t* pool_begin,
                                    const int32_t* pool_end, int32_t max_pools, uint16_t* pools, hipStream_t s);
hipError_t launch_scores_with_groups_paged(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                           const uint16_t* pools, const int32_t* first_valid, const int32_t* table,
                                           int32_t table_stride, int32_t num_seqs, const int32_t* q_seq,
                                           const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                           hipStream_t s);
hipError_t launch_topk_groups_paged(const dsa_dims& d, const float* scores, int32_t stride, const int32_t* first_valid,
                                    const int32_t* table, int32_t table_stride, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                                    const void* ws, hipStream_t s);

// INT8 pools (code rows of idx_dim bytes and one fp32 scale per pool).
hipError_t launch_index_pools_int8(const dsa_dims& d, const void* k, const void* gate, int dtype,
                                   const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                   const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                   int8_t* codes, float* scales, float* pools_f32, hipStream_t s);
hipError_t launch_index_scores_int8(const dsa_dims& d, const uint16_t* q_idx, const float* w, const int8_t* codes,
                                    const float* scales, const dsa_seqs& seqs, int32_t num_seqs, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t T, int32_t stride, float* scores, hipStream_t s);
hipError_t launch_scores_with_groups_int8(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                          const int8_t* codes, const float* scales, const dsa_seqs& seqs,
                                          int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                          int32_t stride, float* scores, void* ws, hipStream_t s);
hipError_t launch_append_scores_groups_int8(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                            const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                            const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                                            int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                                            int32_t max_pools, int8_t* codes, float* scales, const uint16_t* q_idx,
                                            const float* w, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                            int32_t stride, float* scores, void* ws, hipStream_t s);

size_t topk_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride);
bool topk_supported(const dsa_dims& d, int32_t stride);
// Rows of at most 40,960 pools are selected in one pass (k_topk_direct, no workspace).
bool topk_direct(int32_t stride);
hipError_t launch_topk(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                       int32_t* indices, void* ws, hipStream_t s);

hipError_t launch_expand(const dsa_dims& d, const int32_t* pool_ids, const dsa_seqs& seqs,
                         const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* indices,
                         hipStream_t s);

struct MlaPlan {
    bool mfma;          // MFMA kernel (bf16 q, latent 512, heads % 16 == 0)
    int head_tiles;     // 16-head tiles per workgroup (MFMA path)
    int head_groups;    // workgroups along the head axis
    int rows_chunk;     // k_mla_rows: list positions per chunk (16 RT NW)
    int chunks_per_split;
    int splits;         // list partitions per query
    size_t ws_bytes;    // partial results (0 when splits == 1)
};
MlaPlan plan_sparse_mla(const dsa_dims& d, int32_t T, int32_t num_splits, int q_dtype);
hipError_t launch_sparse_mla(const dsa_dims& d, const MlaPlan& plan, const void* q, int q_dtype,
                             const int8_t* cache, const int32_t* indices, int32_t T, float scale,
                             void* out, int out_dtype, float* lse, void* ws, hipStream_t s);

// The merge of a split plan's partials (nothing when plan.splits == 1).
hipError_t launch_mla_merge(const dsa_dims& d, const MlaPlan& plan, int32_t T, void* ws, void* out, int out_dtype,
                            float* lse, hipStream_t s);
// Selection from the group lists, the expanded list and the split attention
// in one launch, then the merge; shapes the one-launch form does not cover
// run launch_topk_groups + launch_sparse_mla.
hipError_t launch_select_mla(const dsa_dims& d, const MlaPlan& plan, const float* scores, int32_t stride,
                             const dsa_seqs& seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                             int32_t* pool_ids, int32_t* indices, const void* sel_ws, const void* q, int q_dtype,
                             const int8_t* cache, float scale, void* out, int out_dtype, float* lse, void* mla_ws,
                             hipStream_t s);

// The device address of the no-allocation entry point's fixed array on the
// current device (resolved once per device).
hipError_t noalloc_scratch(void** out);

bool decode_step_supported(const dsa_dims& d, int32_t T, int32_t stride);
size_t decode_step_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride);
hipError_t launch_decode_step(const dsa_dims& d, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                              const dsa_seqs& seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                              int32_t stride, const uint16_t* q, const int8_t* cache, float scale, void* out,
                              int out_dtype, float* lse, int32_t* pool_ids, int32_t* indices, void* ws,
                              hipStream_t s);

}  // namespace dsa_host
