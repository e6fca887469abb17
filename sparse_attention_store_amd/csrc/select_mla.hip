// topk_select over the scoring pass's group lists, expand_selection and the
// split attention of sparse_mla in one launch ([Ref] Functions:
// topk_pools, expand_selection, mla_masked_attention; [Kernels] Included
// and Install: split-KV decode over one shared INT8 latent).
//
// k_select_mla<NW> is k_mla_rows<1, NW> with the list computed in place:
// every attention workgroup of a query first makes the query's selection
// from the group lists itself (select_from_groups on its 64 NW threads; the
// 17 workgroups of a query repeat the same work, which costs less than a
// kernel boundary and a dependent read of the index list), then takes its
// chunk's cache rows from the ids in LDS.  Workgroup (split 0, head group 0)
// also writes pool_ids and the index list.  The selection state and the
// attention's staging share LDS: the selection is done before the
// attention's first LDS write, and the ids sit outside the shared part.
// The partials are merged by k_mla_combine, as in sparse_mla.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "group_select.h"
#include "mla_core.h"

namespace dsa {

template <int NW>
struct SelectMlaSmem {
    int32_t sel[kGroupMaxK];
    union {
        GroupSelCore<64 * NW> g;
        MlaRowsSmemT<1, NW> m;
    } u;
};

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_select_mla(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int stride, int select_k, const uint64_t* __restrict__ cand,
    const int32_t* __restrict__ cand_n, Emit e, const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache,
    int row_bytes, int H, float scale_log2, int chunks_per_split, int splits, float* __restrict__ part_o,
    MlaPartial* __restrict__ part_ml, void* __restrict__ out, int out_f32, float* __restrict__ lse) {
    constexpr int NT = 64 * NW, CH = 16 * NW;
    __shared__ __attribute__((aligned(16))) SelectMlaSmem<NW> sm;
    const int split = blockIdx.x, t = blockIdx.z, head0 = blockIdx.y * 16;
    // q is read right behind the group lists, so that it has arrived when
    // the attention starts
    constexpr int QP = 16 * kD * 2 / 16 / NT;
    u32x4 qv[QP];
    const GroupQuery g = select_from_groups<NT>(sm.u.g, sm.sel, scores, first_valid, q_seq, q_pos, e.row_base,
                                                stride, select_k, cand, cand_n, t, [&] {
#pragma unroll
                                                    for (int i = 0; i < QP; ++i)
                                                        qv[i] = mla_q_piece<NT>(q, t, H, head0, i);
                                                }, [&] { mla_stage_q<NT>(sm.u.m.qs, qv); });
    if (!g.listed) {                                // no barrier was taken: stage q now
        mla_stage_q<NT>(sm.u.m.qs, qv);
        lds_barrier();
    }
    const int32_t* sel = g.listed ? sm.sel : nullptr;
    if (split == 0 && blockIdx.y == 0) emit_selection<NT>(sel, g.K, select_k, t, g.b, g.f, g.qp, g.n_vis, e, g.rb);
    // list position -> cache row, exactly as emit_selection writes it
    const int64_t base = g.rb + g.f;
    const int nsel = 4 * g.K;
    const int tail = g.qp >= g.f ? (g.qp - g.f + 1) - 4 * g.n_vis : 0;
    const int n_vis = g.n_vis;
    auto idx_at = [&](int pos) -> int {
        int64_t v = -1;
        if (pos < nsel) v = base + 4 * (int64_t)(sel ? sel[pos >> 2] : (pos >> 2)) + (pos & 3);
        else if (pos < nsel + tail) v = base + 4 * (int64_t)n_vis + (pos - nsel);
        return (int32_t)v;
    };
    const int W = e.W;
    const int nchunks = (W + CH - 1) / CH;
    const int c_begin = split * chunks_per_split;
    const int c_end = min(c_begin + chunks_per_split, nchunks);
    mla_rows_split<1, false, NW, true>(sm.u.m, [&](int i) { return qv[i]; }, cache, row_bytes, idx_at, W, H, scale_log2, t,
                                 head0, split, c_begin, c_end, splits, part_o, part_ml, out, out_f32, lse);
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_select_mla(const dsa_dims& d, const MlaPlan& plan, const float* scores, int32_t stride,
                             const dsa_seqs& seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                             int32_t* pool_ids, int32_t* indices, const void* sel_ws, const void* q, int q_dtype,
                             const int8_t* cache, float scale, void* out, int out_dtype, float* lse, void* mla_ws,
                             hipStream_t s) {
    if (T == 0) return hipSuccess;
    constexpr int NW = 8;
    static_assert(16 * NW == dsa::kRChunk, "the attention walks kRChunk-row chunks");
    if (!(plan.mfma && plan.head_tiles == 1 && plan.rows_chunk == dsa::kRChunk)) {
        hipError_t e = launch_topk_groups(d, scores, stride, seqs, q_seq, q_pos, T, pool_ids, indices, sel_ws, s);
        if (e != hipSuccess) return e;
        return launch_sparse_mla(d, plan, q, q_dtype, cache, indices, T, scale, out, out_dtype, lse, mla_ws, s);
    }
    const uint64_t* cand = reinterpret_cast<const uint64_t*>(sel_ws);
    const int32_t* cand_n = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(sel_ws) +
                                                             ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256);
    const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
    const int H = d.mla_heads;
    float* part_o = reinterpret_cast<float*>(mla_ws);
    dsa::MlaPartial* part_ml = nullptr;
    if (plan.splits > 1)
        part_ml = reinterpret_cast<dsa::MlaPartial*>(part_o + (size_t)T * plan.splits * H * dsa::kD);
    dim3 grid((unsigned)plan.splits, (unsigned)plan.head_groups, (unsigned)T);
    hipLaunchKernelGGL((dsa::k_select_mla<NW>), grid, dim3(64 * NW), 0, s, scores, seqs.first_valid, q_seq, q_pos,
                       stride, d.index_topk / d.kpool, cand, cand_n, e, reinterpret_cast<const uint16_t*>(q),
                       reinterpret_cast<const uint8_t*>(cache), d.row_bytes, H, scale * dsa::kLog2e,
                       plan.chunks_per_split, plan.splits, part_o, part_ml, out, out_dtype == DSA_F32 ? 1 : 0, lse);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_mla_merge(d, plan, T, mla_ws, out, out_dtype, lse, s);
}

}  // namespace dsa_host
