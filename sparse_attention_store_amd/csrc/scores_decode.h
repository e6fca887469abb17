// Definitions shared by the decode scoring kernels (k_scores_groups in
// index_scores.hip, k_scores_runs in index_scores_runs.hip): the step's
// new-token arguments and the host helpers that fill them.
#pragma once
#include <algorithm>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "scores_core.h"
#include "topk_core.h"

namespace dsa {

constexpr int kDecMaxT = 64;
constexpr int kQStride = kDI + 8;          // bf16 per LDS row of the shared A operand
struct AppendArgs {    // the step's new tokens (append_tokens' arguments)
    const uint16_t* latent;
    int64_t n, ld;
    const int64_t* slots;
    int8_t* cache;
    int row_bytes;
    const uint16_t* k;
    const uint16_t* gate;
    const float* ln_w;
    const float* ln_b;
    float eps;
    const int64_t* tok_base;
    const int32_t* pool_begin;
    const int32_t* pool_end;
    uint16_t* pools;   // the same buffer the tiles read (bf16 pools, or the INT8 code rows,
                       // whose scales are the kernel's pool_scales)
    int pool_bx;       // 4-pool blocks per sequence (0: no pools)
    int pool_tasks;    // num_seqs * pool_bx
    int tasks;         // pool_tasks + ceil(n / 4)
};

}  // namespace dsa

namespace dsa_host {

// Events of the next timed scoring launch (time_next_scoring_launch), taken once.
void take_events(hipEvent_t& a, hipEvent_t& b);

// The group lists in a scoring workspace: T x kGroupCandCap entries, then T x
// kMaxGroups counts.
inline void group_lists(void* ws, int32_t T, uint64_t*& cand, int32_t*& cand_n) {
    cand = reinterpret_cast<uint64_t*>(ws);
    cand_n = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                        ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256);
}

// The new tokens' part of a fused launch (dsa_append_tokens' arguments); for
// INT8 pools, the code rows take the bf16 pool buffer's place (the scales are
// the kernel's pool_scales argument).
inline bool make_append_args(const dsa_dims& d, const void* latent, int64_t n, int64_t ld, const int64_t* slots,
                      int8_t* cache, const void* k, const void* gate, const float* ln_w, const float* ln_b,
                      const dsa_seqs& seqs, int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                      int32_t max_pools, uint16_t* pools, int8_t* codes, dsa::AppendArgs& ap) {
    ap = dsa::AppendArgs{};
    ap.latent = reinterpret_cast<const uint16_t*>(latent);
    ap.n = n;
    ap.ld = ld;
    ap.slots = slots;
    ap.cache = cache;
    ap.row_bytes = d.row_bytes;
    ap.k = reinterpret_cast<const uint16_t*>(k);
    ap.gate = reinterpret_cast<const uint16_t*>(gate);
    ap.ln_w = ln_w;
    ap.ln_b = ln_b;
    ap.eps = d.ln_eps;
    ap.tok_base = seqs.tok_base;
    ap.pool_begin = pool_begin;
    ap.pool_end = pool_end;
    ap.pools = pools ? pools : reinterpret_cast<uint16_t*>(codes);
    ap.pool_bx = max_pools > 0 ? (int)cdiv(max_pools, 4) : 0;
    const int64_t pool_tasks = (int64_t)ap.pool_bx * num_seqs;   // 0 without pools
    const int64_t tasks = pool_tasks + cdiv(n, 4);
    if (tasks > 0x3FFFFFFF) return false;
    ap.pool_tasks = (int)pool_tasks;
    ap.tasks = (int)tasks;
    return true;
}

inline unsigned fused_grid(int32_t T, int32_t stride, int tasks) {
    const int64_t want = cdiv(cdiv(stride, dsa::kGroupPools), 4) * (int64_t)T + tasks;
    return (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 4 * (int64_t)device_info().cu_count);
}


}  // namespace dsa_host
