// Decode scoring for runs of queries that share one pass over their
// sequence's pools (dsa_append_scores_groups_shared).
#include <hip/hip_ext.h>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "scores_core.h"
#include "topk_core.h"
#include "new_tokens.h"
#include "scores_decode.h"

namespace dsa {

// k_scores_runs: k_scores_groups for queries that share one pass over the
// pools.  Consecutive queries of one sequence (e.g. the 1 + 3 tokens of a
// speculative decode step, [Flash] Deployment target and Stream C:
// indexer_share_mtp) form runs of at most `share` (<= R); a tile's pool rows
// are loaded once and scored for every query of its run, each against its own
// visible count, so the pools are read once per run instead of once per
// query.  Each query's scores, group lists and -inf tail are the bits it gets
// from k_scores_groups alone (the same per-query operations, the same
// operands).  The queries' A operands of a tile go through LDS one after the
// other; the kernel runs 2 workgroups per CU (it needs more registers than the
// one-query kernel, and 8 waves per CU still keep far more pool loads in
// flight than HBM needs).
constexpr int kShare = 4;
struct RunGeom {
    // per run (valid at the run's first query)
    int64_t base;      // pool_base of the run's sequence
    uint32_t first;    // flat index of the run's first tile
    uint32_t ntiles;   // 256-pool tiles of the run's visible pools (largest visible count of its queries)
    int32_t ng;        // 64-pool groups of those
    int32_t nn;        // that largest visible count, capped at the row stride
    int64_t tok0;      // with new tokens: the sequence's first pooled token row
    int32_t pb, pe;    // with new tokens: the pools this step completes
    int16_t rank;      // with new tokens: rank among the runs that have tiles
    int16_t nq;        // queries in the run (0 for a query that does not start one)
    // per query
    int32_t nnq;       // this query's visible pools, capped at the row stride
};
//
// With I8 the pools are INT8 code rows with one fp32 scale each
// (score_pool_group_i8): each wave loads 8 KB of codes and its pools' scales,
// and a rebuilt pool is quantised the way the pool tasks store it.
template <bool CANDS, int AD, bool I8 = false, int R = kShare>
__global__ __launch_bounds__(256, 2) void k_scores_runs(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const void* pools_v, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int T, int nseq, int stride, float* __restrict__ scores,
    int select_k, uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n, AppendArgs ap,
    float* pool_scales, int share) {
    __shared__ RunGeom geom[kDecMaxT];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[R][kHI * kQStride];
    __shared__ __attribute__((aligned(16))) float s_w[R][kHI];
    __shared__ __attribute__((aligned(16))) uint32_t s_new[AD ? 4 : 1][kDI / 2];
    const uint16_t* pools = reinterpret_cast<const uint16_t*>(pools_v);
    const int8_t* codes = reinterpret_cast<const int8_t*>(pools_v);
    const int lane = threadIdx.x & 63;
    const int wave = uniform32(threadIdx.x >> 6);
    if (wave == 0) {
        // One memory round trip: lane t < T reads query t's fields while lane
        // s < nseq reads sequence s's (bounded buffer loads: absent fields
        // read 0), then each query takes its sequence's from that lane.  With
        // more than 64 sequences they are read by query, after q_seq.
        const bool pools_ad = AD && ap.pool_bx > 0;
        const uint32_t l4 = (uint32_t)lane * 4u;
        const uint32_t qb = (uint32_t)min(T, kWave) * 4u;
        const int b = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(q_seq, qb), l4, 0, 0);
        const int qp = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(q_pos, qb), l4, 0, 0);
        const uint32_t sb = (uint32_t)nseq * 4u, pbb = pools_ad ? sb : 0u;
        int f, pb_s, pe_s;
        u32x2 bs, ts;
        auto fields = [&](uint32_t s4) {
            f = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(first_valid, sb), s4, 0, 0);
            bs = __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(pool_base, 2u * sb), 2u * s4, 0, 0);
            pb_s = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ap.pool_begin, pbb), s4, 0, 0);
            pe_s = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ap.pool_end, pbb), s4, 0, 0);
            ts = __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(ap.tok_base, 2u * pbb), 2u * s4, 0, 0);
        };
        if (nseq <= kWave) {
            fields(l4);                                 // independent of b: issued with the query loads
            f = __shfl(f, b);
            bs[0] = (uint32_t)__shfl((int)bs[0], b);
            bs[1] = (uint32_t)__shfl((int)bs[1], b);
            pb_s = __shfl(pb_s, b);
            pe_s = __shfl(pe_s, b);
            ts[0] = (uint32_t)__shfl((int)ts[0], b);
            ts[1] = (uint32_t)__shfl((int)ts[1], b);
        } else {
            fields((uint32_t)b * 4u);
        }
        const bool act = lane < T;
        int nn = 0, pb = 0, pe = 0;
        int64_t base = 0, tok0 = 0;
        if (act) {
            nn = min(qp >= f ? (qp - f + 1) >> 2 : 0, stride);
            base = (int64_t)(((uint64_t)bs[1] << 32) | bs[0]);
            if (pools_ad) {
                pb = pb_s;
                pe = min(pe_s, pb + 4 * ap.pool_bx);          // what the pool tasks build
                tok0 = (int64_t)(((uint64_t)ts[1] << 32) | ts[0]) + f;
            }
        }
        // Runs: a query starts one where the sequence changes, and every
        // `share` queries along a longer stretch of one sequence.
        const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
        bool brk = act && (lane == 0 || __shfl(b, lane > 0 ? lane - 1 : 0) != b);
        if constexpr (R > 1) {
            const uint64_t m0 = __ballot(brk) & upto;
            const int ps = m0 ? 63 - __clzll((long long)m0) : 0;
            brk = act && (lane - ps) % share == 0;
        }
        const uint64_t starts = __ballot(brk);
        const uint64_t later = starts & ~upto;
        const int nq = brk ? min(later ? __ffsll((long long)later) - 1 : T, T) - lane : 0;
        int nn_run = nn;
#pragma unroll
        for (int i = 1; i < R; ++i) {
            const int o = __shfl(nn, min(lane + i, 63));
            if (i < nq) nn_run = max(nn_run, o);
        }
        const int ng = brk ? (nn_run + kGroupPools - 1) / kGroupPools : 0;
        uint32_t nt = (uint32_t)(ng + 3) >> 2;
        // With new tokens, every run's last tile (the one holding the pools
        // the step completes, which its waves rebuild) comes first, in query
        // order, so that extra work is done early, not in the launch's tail;
        // the other tiles follow.  `first`/`ntiles` then describe those others.
        const unsigned long long lead = __ballot(nt > 0);
        const int rank = nt > 0 ? popc_below(lead) : -1;
        uint32_t off = 0;
        if constexpr (AD != 0) {
            nt = nt > 0 ? nt - 1 : 0;
            off = (uint32_t)__popcll(lead);
        }
        const uint32_t incl = wave_incl_sum_u32(nt);
        geom[lane] = RunGeom{base, off + incl - nt, nt, ng, nn_run, tok0, pb, pe, (int16_t)rank, (int16_t)nq, nn};
    }
    lds_barrier();
    const int total = (int)(geom[63].first + geom[63].ntiles);
    int tile = blockIdx.x;
    for (; tile < total; tile += gridDim.x) {
        int t, j;
        if (AD != 0 && tile < (int)uniform32((int)geom[0].first)) {
            t = __ffsll((long long)__ballot(geom[lane].rank == tile)) - 1;   // the tile-th run's last tile
            j = (uniform32(geom[t].ng) - 1) >> 2;
        } else {
            // the run of the tile: the number of queries whose tiles all come before it
            t = __popcll(__ballot(geom[lane].first + geom[lane].ntiles <= (uint32_t)tile));
            j = tile - uniform32((int)geom[t].first);
        }
        const int nq = R > 1 ? uniform32(geom[t].nq) : 1;
        const int grp = 4 * j + wave;
        const bool has = grp < uniform32(geom[t].ng);
        const int n_vis = uniform32(geom[t].nn);
        const int p0 = grp * kGroupPools;
        // The A operands of the run's queries: wave w loads heads 8 w .. 8 w + 7
        // of each (two 16-byte pieces per lane), plus the head weights; issued
        // before the pool rows.  (Buffer loads: the lane part of each address
        // is a 32-bit offset.)
        u32x4 qv[R][2];
        float wt[R];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            if (m < nq) {
                const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q_idx + (int64_t)(t + m) * (kHI * kDI), kHI * kDI * 2);
                const uint32_t loff = (uint32_t)((lane >> 4) * (kDI * 2) + (lane & 15) * 16);
#pragma unroll
                for (int i = 0; i < 2; ++i)          // piece lane + 64 i: head 8 w + 4 i + lane / 16, dims 8 (lane % 16) ..
                    qv[m][i] = ld_buf128(rq, loff, (uint32_t)((8 * wave + 4 * i) * (kDI * 2)));
                wt[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    buffer_rsrc(w + (int64_t)(t + m) * kHI, kHI * 4), (uint32_t)min(lane, 7) * 4u, (uint32_t)(32 * wave),
                    0));
            }
        }
        // A wave past the run's last group re-reads the tile's first row
        // (unconditional loads keep the wait counts exact).
        u32x4 v[I8 ? 8 : 16];
        float psc = 0.f;                               // INT8: the scale of pool p0 + lane
        const int lp0 = has ? p0 : p0 - kGroupPools * wave;
        {
            const int64_t row0 = (int64_t)uniform64((uint64_t)geom[t].base) + lp0;
            const int lim = has ? n_vis - p0 : 1;
            if constexpr (I8) {
                load_pool_group_i8(codes + row0 * kDI, lim, v);
                psc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    buffer_rsrc(pool_scales + row0, (uint32_t)(min(lim, 64) * 4)), (uint32_t)min(lane, lim - 1) * 4u,
                    0, 0));
            } else {
                load_pool_group(pools + row0 * kDI, lim, v);
            }
        }
        __builtin_amdgcn_sched_barrier(0);             // every load in flight before the A operands are shared
        // the group list lengths, while the rows are in flight
        int gm[R];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int nv = R > 1 ? uniform32(geom[t + (m < nq ? m : 0)].nnq) : n_vis;
            gm[m] = CANDS && nv > select_k ? group_quota<true>(select_k, nv) : 0;
        }
#pragma unroll
        for (int m = 0; m < R; ++m) {
            if (m < nq) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int k = lane + 64 * i;
                    *reinterpret_cast<u32x4*>(&s_q[m][(8 * wave + (k >> 4)) * kQStride + 8 * (k & 15)]) = qv[m][i];
                }
                if (lane < 8) s_w[m][8 * wave + lane] = wt[m];
            }
        }
        lds_barrier();
        if (has) {
            float sv[R];
#pragma unroll
            for (int m = 0; m < R; ++m) {
                sv[m] = 0.f;
                if (R > 1) __builtin_amdgcn_sched_barrier(0);   // one member's operand at a time
                if (m < nq) {
                    if constexpr (I8) {
                        IdxQueryI8 Q;
                        load_idx_query_lds_i8(s_q[m], kQStride, s_w[m], Q);
                        sv[m] = score_pool_group_i8(Q, v, psc);
                    } else {
                        IdxQuery Q;
                        load_idx_query_lds(s_q[m], kQStride, s_w[m], Q);
                        sv[m] = score_pool_group(Q, v);
                    }
                }
            }
            if constexpr (AD != 0) {
                // Completed pools are rebuilt with the pool tasks' code into
                // s_new[wave] and scored as a single column (lane pp - p0 gets
                // the bits the group's own scoring would have given it).
                const int nb = max(uniform32(geom[t].pb), p0);
                const int ne = min(min(uniform32(geom[t].pe), p0 + kGroupPools), n_vis);
                const int64_t tok0 = (int64_t)uniform64((uint64_t)geom[t].tok0);
                for (int pp = nb; pp < ne; ++pp) {
                    PoolRaw128 r;
                    pool_raw_load(ap.k, ap.gate, tok0 + 4 * (int64_t)pp, r);
                    PoolIn<kDI, uint16_t> in;
                    pool_raw_in(r, in);
                    if constexpr (I8) {
                        // the INT8 form: the pool tasks' values and quantiser,
                        // the codes through s_new[wave] as 128 bytes
                        float f[2];
                        pool_values_f32<kDI, uint16_t>(in, ap.ln_w, ap.ln_b, ap.eps, f);
                        int8_t code[2];
                        const float sc = quantize_pool<2>(f, code);
                        reinterpret_cast<uint16_t*>(s_new[wave])[lane] =
                            (uint16_t)((uint8_t)code[0] | ((uint32_t)(uint8_t)code[1] << 8));
                        wave_lds_fence();
                        const char* nbytes = reinterpret_cast<const char*>(s_new[wave]) + 32 * (lane >> 4);
                        const u32x4 w0 = *reinterpret_cast<const u32x4*>(nbytes);
                        const u32x4 w1 = *reinterpret_cast<const u32x4*>(nbytes + 16);
#pragma unroll
                        for (int m = 0; m < R; ++m) {
                            if (R > 1) __builtin_amdgcn_sched_barrier(0);
                            if (m < nq) {
                                IdxQueryI8 Q2;         // reloaded: Q is not kept through the rebuild
                                load_idx_query_lds_i8(s_q[m], kQStride, s_w[m], Q2);
                                const float s2 = score_pool_column_i8(Q2, w0, w1, sc);
                                if (lane == pp - p0) sv[m] = s2;
                            }
                        }
                    } else {
                        uint16_t ov[2];
                        pool_values<kDI, uint16_t>(in, ap.ln_w, ap.ln_b, ap.eps, ov);
                        s_new[AD ? wave : 0][lane] = (uint32_t)ov[0] | ((uint32_t)ov[1] << 16);
                        wave_lds_fence();
                        const int g = lane >> 4;
                        u32x4 nb4[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            nb4[i] = *reinterpret_cast<const u32x4*>(&s_new[AD ? wave : 0][16 * i + 4 * g]);
#pragma unroll
                        for (int m = 0; m < R; ++m) {
                            if (R > 1) __builtin_amdgcn_sched_barrier(0);
                            if (m < nq) {
                                IdxQuery Q2;           // reloaded: Q is not kept through the rebuild
                                load_idx_query_lds(s_q[m], kQStride, s_w[m], Q2);
                                const float s2 = score_pool_column(Q2, nb4);
                                if (lane == pp - p0) sv[m] = s2;
                            }
                        }
                    }
                    wave_lds_fence();                  // s_new is rewritten by the next pool
                }
            }
            const int p = p0 + lane;
#pragma unroll
            for (int m = 0; m < R; ++m) {
                if (R > 1) __builtin_amdgcn_sched_barrier(0);
                if (m < nq) {
                    const int tq = t + m;
                    const int nv = R > 1 ? uniform32(geom[tq].nnq) : n_vis;
                    {
                        // a buffer store: pools at or past the row stride fall outside its range
                        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scores + (int64_t)tq * stride + p0,
                                                                      (uint32_t)(min(stride - p0, kGroupPools) * 4));
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p < nv ? sv[m] : -INFINITY), rs,
                                                              (uint32_t)lane * 4u, 0, 0);
                    }
                    if constexpr (CANDS) {
                        // only the query's own groups (a shorter query of the run has fewer)
                        if (nv > select_k && p0 < nv)
                            keep_group_best(sv[m], p < nv, p, grp, gm[m],
                                            cand + (int64_t)tq * kGroupCandCap, cand_n + (int64_t)tq * kMaxGroups,
                                            [](uint64_t* q, uint64_t x) { *q = x; },
                                            [](int32_t* q, uint32_t x) { *q = (int32_t)x; });
                    }
                }
            }
        }
        if (tile + (int)gridDim.x < total) lds_barrier();   // s_q is rewritten by the next tile
    }
    if constexpr (AD != 0) {
        // New tokens: tasks total .. total + tasks - 1, 4 pools or 4 rows each.
        for (; tile < total + ap.tasks; tile += gridDim.x) {
            const int a = tile - total;
            if (a < ap.pool_tasks) {
                if constexpr (I8)
                    index_pool_row_int8<kDI, uint16_t>(ap.k, ap.gate, ap.ln_w, ap.ln_b, ap.eps, first_valid,
                                                       ap.tok_base, pool_base, ap.pool_begin, ap.pool_end,
                                                       PoolDst{nullptr, reinterpret_cast<int8_t*>(ap.pools),
                                                               pool_scales, nullptr},
                                                       a / ap.pool_bx, (a % ap.pool_bx) * 4 + wave);
                else
                    index_pool_row<kDI, uint16_t>(ap.k, ap.gate, ap.ln_w, ap.ln_b, ap.eps, first_valid, ap.tok_base,
                                                  pool_base, ap.pool_begin, ap.pool_end, ap.pools, a / ap.pool_bx,
                                                  (a % ap.pool_bx) * 4 + wave);
            } else
                store_int8_row<AD, false>(ap.latent, ap.n, ap.ld, ap.slots, ap.cache, ap.row_bytes,
                                          (int64_t)(a - ap.pool_tasks) * 4 + wave);
        }
    }
    // Pools past each query's last visible group: written by the workgroups
    // that had neither a tile nor a task when there are such, so that the
    // waves finishing the last tiles have nothing more to do.
    const int busy = total + (AD != 0 ? ap.tasks : 0);
    const int first = busy < (int)gridDim.x ? busy : 0;
    if ((int)blockIdx.x < first) return;
    const int gw = ((int)blockIdx.x - first) * 4 + wave, W = ((int)gridDim.x - first) * 4;
    for (int t = 0; t < T; ++t) {
        const int from = (geom[t].nnq + kGroupPools - 1) / kGroupPools * kGroupPools;
        float* out = scores + (int64_t)t * stride;
        for (int p = from + gw * kGroupPools + lane; p < stride; p += W * kGroupPools) out[p] = -INFINITY;
    }
}

}  // namespace dsa

namespace dsa_host {

// ------------------------------------------------------------------ shared runs

hipError_t launch_append_scores_groups_runs(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                            const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                            const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                                            int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                                            int32_t max_pools, void* pools, float* scales, const uint16_t* q_idx,
                                            const float* w, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                            int32_t stride, float* scores, void* ws, int share, hipStream_t s) {
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    dsa::AppendArgs ap;
    const bool i8 = scales != nullptr;
    if (!make_append_args(d, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, seqs, num_seqs, pool_begin, pool_end,
                          max_pools, i8 ? nullptr : reinterpret_cast<uint16_t*>(pools),
                          i8 ? reinterpret_cast<int8_t*>(pools) : nullptr, ap))
        return hipErrorInvalidValue;
    const bool tokens = n > 0 || max_pools > 0;
    const int64_t want = cdiv(cdiv(stride, dsa::kGroupPools), 4) * (int64_t)T + ap.tasks;
    const unsigned grid =
        (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 2 * (int64_t)device_info().cu_count);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
#define DSA_RUNS(D, I8)                                                                                              \
    hipExtLaunchKernelGGL((dsa::k_scores_runs<true, D, I8>), dim3(grid), dim3(256), 0, s, ev0, ev1, 0, q_idx, w,   \
                          pools, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, num_seqs, stride, scores,    \
                          d.index_topk / d.kpool, cand, cand_n, ap, scales, share)
#define DSA_RUNS_D(I8)                                       \
    if (!tokens) { DSA_RUNS(0, I8); } else switch (d.latent_dim) { \
        case 512: DSA_RUNS(512, I8); break;                  \
        case 256: DSA_RUNS(256, I8); break;                  \
        case 128: DSA_RUNS(128, I8); break;                  \
        default: DSA_RUNS(64, I8); break;                    \
    }
    if (i8) { DSA_RUNS_D(true) } else { DSA_RUNS_D(false) }
#undef DSA_RUNS_D
#undef DSA_RUNS
    return hipGetLastError();
}

}  // namespace dsa_host
