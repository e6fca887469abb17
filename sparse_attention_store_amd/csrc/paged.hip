// The path's calls over paged caches (paged.h): pool building and the
// selection with its expanded index list; scoring over paged pools is
// k_scores_groups<.., PAGED> (index_scores.hip), and the attention takes the
// index list, whose entries are then physical rows.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "group_select.h"
#include "new_tokens.h"
#include "paged.h"
#include "topk_core.h"

namespace dsa {

// Pool pool_begin[b] + j of sequence b (one wave): as index_pool_row, with
// each of the pool's kpool token rows and the pool's row taken through the
// block table (the four tokens of a pool can straddle a block when the left
// padding is not a multiple of 4).
template <int DI, typename T>
__global__ __launch_bounds__(256) void k_index_pools_paged(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid, PagedMap pm,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end, uint16_t* __restrict__ pools) {
    constexpr int KP = PoolIn<DI, T>::KP, CPL = PoolIn<DI, T>::CPL;
    const int b = blockIdx.y, lane = threadIdx.x & 63;
    const int p = pool_begin[b] + (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (p >= pool_end[b]) return;
    const int64_t x0 = (int64_t)first_valid[b] + 4 * (int64_t)p;
    const bool active = DI >= 64 || lane < DI;
    const int c0 = active ? lane * CPL : 0;
    PoolIn<DI, T> in;
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        const int64_t row = pm.row(b, x0 + s);
        const T* kr = k + row * DI + c0;
        const T* gr = gate + row * DI + c0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            in.x[s][c] = active ? load_val<T>(kr + c) : 0.f;
            in.g[s][c] = active ? load_val<T>(gr + c) : 0.f;
        }
    }
    uint16_t outv[CPL];
    pool_values<DI, T>(in, ln_w, ln_b, eps, outv);
    if (!active) return;
    uint16_t* dst = pools + pm.pool_row(b, p) * (int64_t)DI + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[c] = outv[c];
}

// k_topk_groups with the index list through the block table: the same
// selection (select_from_groups), then pool ids and the rows of each selected
// pool's positions and of the visible tail, -1 filled ([Ref] Functions:
// topk_pools, expand_selection).
__global__ __launch_bounds__(1024) void k_topk_groups_paged(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int stride, int select_k, const uint64_t* __restrict__ cand,
    const int32_t* __restrict__ cand_n, PagedMap pm, int32_t* __restrict__ pool_ids, int32_t* __restrict__ indices,
    int W) {
    constexpr int NT = 1024;
    static_assert(NT == kMaxGroups, "one group count per thread");
    __shared__ GroupSelCore<NT> G;
    __shared__ int32_t sel[kGroupMaxK];
    const int t = blockIdx.x, tid = threadIdx.x;
    const GroupQuery g = select_from_groups<NT>(G, sel, scores, first_valid, q_seq, q_pos, nullptr, stride, select_k,
                                                cand, cand_n, t, [] {}, [] {});
    const int32_t* sl = g.listed ? sel : nullptr;
    if (pool_ids) {
        int32_t* out = pool_ids + (int64_t)t * select_k;
        for (int i = tid; i < select_k; i += NT) out[i] = i < g.K ? (sl ? sl[i] : i) : -1;
    }
    const int nsel = 4 * g.K;
    const int tail = g.qp >= g.f ? (g.qp - g.f + 1) - 4 * g.n_vis : 0;
    int32_t* out = indices + (int64_t)t * W;
    for (int j = tid; j < W; j += NT) {
        int64_t x = -1;
        if (j < nsel) x = g.f + 4 * (int64_t)(sl ? sl[j >> 2] : (j >> 2)) + (j & 3);
        else if (j < nsel + tail) x = g.f + 4 * (int64_t)g.n_vis + (j - nsel);
        out[j] = x >= 0 ? (int32_t)pm.row(g.b, x) : -1;
    }
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_index_pools_paged(const dsa_dims& d, const void* k, const void* gate, int dtype, const float* ln_w,
                                    const float* ln_b, const int32_t* first_valid, const int32_t* table,
                                    int32_t table_stride, int32_t num_seqs, const int32_t* pool_begin,
                                    const int32_t* pool_end, int32_t max_pools, uint16_t* pools, hipStream_t s) {
    if (max_pools <= 0 || num_seqs <= 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(max_pools, 4), (unsigned)num_seqs), block(256);
    const dsa::PagedMap pm{table, table_stride};
#define DSA_POOLS_PAGED(DI, T)                                                                                   \
    hipLaunchKernelGGL((dsa::k_index_pools_paged<DI, T>), grid, block, 0, s, (const T*)k, (const T*)gate, ln_w,  \
                       ln_b, d.ln_eps, first_valid, pm, pool_begin, pool_end, pools)
    if (d.idx_dim == 128) {
        if (dtype == DSA_F32) DSA_POOLS_PAGED(128, float); else DSA_POOLS_PAGED(128, uint16_t);
    } else {
        if (dtype == DSA_F32) DSA_POOLS_PAGED(32, float); else DSA_POOLS_PAGED(32, uint16_t);
    }
#undef DSA_POOLS_PAGED
    return hipGetLastError();
}

hipError_t launch_topk_groups_paged(const dsa_dims& d, const float* scores, int32_t stride, const int32_t* first_valid,
                                    const int32_t* table, int32_t table_stride, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                                    const void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const uint64_t* cand = reinterpret_cast<const uint64_t*>(ws);
    const int32_t* cand_n = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(ws) +
                                                             ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256);
    hipLaunchKernelGGL(dsa::k_topk_groups_paged, dim3((unsigned)T), dim3(1024), 0, s, scores, first_valid, q_seq, q_pos,
                       stride, d.index_topk / d.kpool, cand, cand_n, dsa::PagedMap{table, table_stride}, pool_ids,
                       indices, d.out_width);
    return hipGetLastError();
}

}  // namespace dsa_host
