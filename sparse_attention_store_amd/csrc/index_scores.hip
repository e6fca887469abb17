// index_scores: score[t][p] = sum_h w[t][h] * relu(q_idx[t][h] . pool[p])
// ([Ref] Functions: index_scores -- matmul, ReLU, head-weighted sum).
//
// MFMA kernel (32 heads x 128): the contraction q_idx[t] (32 x 128) x
// pool^T (128 x pools) maps onto v_mfma_f32_32x32x16_bf16 with the 32 heads
// as M and 32 pools per N-tile.  Each wave keeps 64 pools (two N-tiles, 64
// VGPRs) resident as the B operand and walks the queries of its workgroup;
// query rows are staged through LDS (padded rows, conflict-free 16-byte
// reads) with a register prefetch of the next batch.  The ReLU and the
// head-weighted sum run on the accumulators: each lane holds 16 heads of one
// pool, the other 16 sit in lane l ^ 32, so one shuffle completes the sum.
// Decode launches one query per workgroup (pure pool streaming, HBM bound);
// prefill launches many queries per workgroup so the resident pools are
// reused (MFMA bound).
#include <hip/hip_ext.h>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "scores_core.h"
#include "topk_core.h"
#include "new_tokens.h"
#include "scores_decode.h"
#include "paged.h"

namespace dsa {

constexpr int kQROW = kDI + 8;                        // padded LDS row (bf16 elements)
constexpr int kQBYTES = kHI * kDI * 2;                // 8 KB per query

//
// With CANDS each wave also keeps, per query, the best pools of its 64-pool
// group (keep_group_best, as the decode kernel does): lane l of a wave holds
// pool p0 + l, so the wave is one group.  The selection then reads the group
// lists (k_topk_groups) instead of sorting 256-pool tiles of the scores.
template <int WAVES, int QB, bool CANDS = false>
__global__ __launch_bounds__(WAVES * 64, CANDS ? 2 : 3) void k_scores_mfma(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ pools, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int T, int q_per_block, int stride,
    float* __restrict__ scores, int select_k, uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n) {
    constexpr int NT = WAVES * 64;
    constexpr int CHUNKS = QB * kQBYTES / 16;              // 16-byte pieces per batch
    constexpr int PER_T = (CHUNKS + NT - 1) / NT;
    __shared__ uint16_t q_lds[QB][kHI * kQROW];
    __shared__ float w_lds[QB][kHI];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int tile0 = blockIdx.x * (WAVES * 64);
    const int p0 = tile0 + wave * 64;
    const int t_begin = blockIdx.y * q_per_block;
    const int t_end = min(T, t_begin + q_per_block);
    if (t_begin >= t_end) return;

    // Register prefetch of one batch of query rows + weights.
    u32x4 pre[PER_T];
    float pre_w = 0.f;
    auto prefetch = [&](int tb) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int c = tid + i * NT;
            const int qi = c / (kQBYTES / 16);
            const int within = c % (kQBYTES / 16);
            const int t = tb + qi;
            if (c < CHUNKS && t < t_end)
                pre[i] = *reinterpret_cast<const u32x4*>(q_idx + (int64_t)t * (kHI * kDI) + within * 8);
        }
        if (tid < QB * kHI) {
            const int t = tb + tid / kHI;
            if (t < t_end) pre_w = w[(int64_t)t * kHI + (tid % kHI)];
        }
    };

    u32x4 breg[2][8];
    int64_t loaded_base = -1;
    int loaded_lim = 0;

    prefetch(t_begin);
    for (int tb = t_begin; tb < t_end; tb += QB) {
        lds_barrier();
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int c = tid + i * NT;
            if (c < CHUNKS) {
                const int qi = c / (kQBYTES / 16);
                const int within = c % (kQBYTES / 16);
                const int r = within >> 4, col = (within & 15) << 3;
                *reinterpret_cast<u32x4*>(&q_lds[qi][r * kQROW + col]) = pre[i];
            }
        }
        if (tid < QB * kHI) w_lds[tid / kHI][tid % kHI] = pre_w;
        lds_barrier();
        if (tb + QB < t_end) prefetch(tb + QB);

        const int nq = min(QB, t_end - tb);
        for (int qi = 0; qi < nq; ++qi) {
            const int t = tb + qi;
            const int b = q_seq[t];
            const int f = first_valid[b];
            const int qp = q_pos[t];
            const int n_vis = qp >= f ? (qp - f + 1) >> 2 : 0;
            float* out = scores + (int64_t)t * stride;
            if (p0 >= n_vis) {                            // whole tile invisible
                const int p = p0 + lane;
                if (p < stride) out[p] = -INFINITY;
                continue;
            }
            const int64_t base = pool_base[b];
            const int lim = min(n_vis - p0, 64);
            if (base != loaded_base || lim > loaded_lim) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int rel = nt * 32 + n;
                    const uint16_t* src = pools + (base + p0 + rel) * kDI + g * 64;
                    const bool ok = rel < lim;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        u32x4 v = {0u, 0u, 0u, 0u};
                        if (ok) v = *reinterpret_cast<const u32x4*>(src + j * 8);
                        breg[nt][j] = v;
                    }
                }
                loaded_base = base;
                loaded_lim = lim;
            }
            f32x16 acc0 = {}, acc1 = {};
            const uint16_t* qrow = &q_lds[qi][n * kQROW + g * 64];
// The 8 A pieces with three reads in flight ahead of the MFMA pairs (the
            // scheduler, short of registers, would otherwise wait on each read
            // right before its pair).
            u32x4 ar[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) ar[j] = *reinterpret_cast<const u32x4*>(qrow + j * 8);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);     // 3 LDS reads
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // 2 MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // 1 LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);     // the last 6 MFMAs
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc0 = mfma32(as_bf16x8(ar[j]), as_bf16x8(breg[0][j]), acc0);
                acc1 = mfma32(as_bf16x8(ar[j]), as_bf16x8(breg[1][j]), acc1);
            }
            // Heads held by this lane: 8*(r/4) + 4*g + (r%4).
            const float* wq = &w_lds[qi][4 * g];
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float wh = wq[8 * (r >> 2) + (r & 3)];
                s0 += wh * relu_bits(acc0[r]);
                s1 += wh * relu_bits(acc1[r]);
            }
            const float sv = add_swap32(s0, s1);           // lanes 0-31: tile 0's sum, 32-63: tile 1's
            const int p = p0 + g * 32 + n;                 // lanes 0-31: tile 0, 32-63: tile 1
            if (p < stride) out[p] = p < n_vis ? sv : -INFINITY;
            if constexpr (CANDS) {
                if (n_vis > select_k)
                    keep_group_best(sv, p < n_vis, p, p0 / kGroupPools, group_quota<true>(select_k, n_vis),
                                    cand + (int64_t)t * kGroupCandCap, cand_n + (int64_t)t * kMaxGroups,
                                    [](uint64_t* q, uint64_t x) { *q = x; },
                                    [](int32_t* q, uint32_t x) { *q = (int32_t)x; });
            }
        }
    }
}

// Decode kernel.  Work is a flat list of 256-pool tiles over the visible
// pools of all queries (a query with ng 64-pool groups has ceil(ng / 4)
// tiles); workgroup tasks are tiles, wave w of a task scores group 4 j + w of
// tile j.  The grid is sized to be resident at once, so every workgroup reads
// the queries' geometry while memory is still idle.  Per tile, the query's
// 8 KB A operand (and its head weights) is loaded once by the workgroup, ahead
// of the pool rows, and shared through LDS (padded rows: conflict-free 16-byte
// reads); each wave loads its group's 16 KB of pool rows straight into MFMA
// B-operand registers, all loads in flight before the first MFMA.  Rows past a
// query's visible count inside its last group, and every pool after that group
// up to the row stride, are written as -inf.
// With CANDS, each wave also keeps its group's best m pools for the selection
// (keep_group_best) when the query has more visible pools than select_k.
//
// With AD (the latent width), the launch also does the step's new tokens
// (the work of append_tokens): after the tiles, tasks of 4 waves store the
// INT8 rows and build the completed pools with the same device code.  Those
// pools may be scored by this very launch while they are being written, so a
// wave whose group holds one rebuilds it from k and gate itself (again the
// same code), puts it into its B-operand registers and scores that; the rows
// it read from memory for it are never used.
struct QueryGeom {
    int64_t base;      // pool_base of the query's sequence
    uint32_t first;    // flat index of the query's first tile
    uint32_t ntiles;   // 256-pool tiles of visible pools
    int32_t ng;        // 64-pool groups of visible pools
    int32_t nn;        // visible pools, capped at the row stride
    int64_t tok0;      // with new tokens: the sequence's first pooled token row
    int32_t pb, pe;    // with new tokens: the pools this step completes
    int32_t rank;      // with new tokens: rank among the queries that have tiles
    int32_t pad;
};
//
// With I8 the pools are INT8 code rows with one fp32 scale each
// (score_pool_group_i8): each wave loads 8 KB of codes and its pools' scales,
// and a rebuilt pool is quantised the way the pool tasks store it.
//
// With PAGED the pools are paged (paged.h): a query's sequence index is kept in
// place of its pool base, and a group's 64 rows are one pool block, found in
// the block table.
//
// With LONG (rows past 65,536 pools), a query of more than 65,536 visible
// pools keeps one list per 256-pool tile: each wave keeps its 64 pools' best
// m in LDS, then wave 0 keeps the best m of those (the best m of the tile are
// among its waves' best m).
template <bool CANDS, int AD, bool I8 = false, bool PAGED = false, bool LONG = false>
__global__ __launch_bounds__(256, 4) void k_scores_groups(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const void* pools_v, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int T, int nseq, int stride, float* __restrict__ scores,
    int select_k, uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n, AppendArgs ap,
    float* pool_scales, PagedMap pm) {
    __shared__ QueryGeom geom[kDecMaxT];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[kHI * kQStride];
    __shared__ __attribute__((aligned(16))) float s_w[kHI];
    __shared__ __attribute__((aligned(16))) uint32_t s_new[AD ? 4 : 1][kDI / 2];
    __shared__ uint64_t s_long[LONG ? 64 : 1];         // the waves' lists of a 256-pool group
    __shared__ int32_t s_long_n[LONG ? 4 : 1];
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
            // (PAGED: no pool bases; the descriptor's range is empty, so nothing is read)
            bs = __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(pool_base, PAGED ? 0u : 2u * sb), 2u * s4, 0, 0);
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
        int nn = 0, pb = 0, pe = 0;
        int64_t base = 0, tok0 = 0;
        if (lane < T) {
            nn = min(qp >= f ? (qp - f + 1) >> 2 : 0, stride);
            base = PAGED ? (int64_t)b : (int64_t)(((uint64_t)bs[1] << 32) | bs[0]);
            if (pools_ad) {
                pb = pb_s;
                pe = min(pe_s, pb + 4 * ap.pool_bx);          // what the pool tasks build
                tok0 = (int64_t)(((uint64_t)ts[1] << 32) | ts[0]) + f;
            }
        }
        const int ng = (nn + kGroupPools - 1) / kGroupPools;
        uint32_t nt = (uint32_t)(ng + 3) >> 2;
        // With new tokens, every query's last tile (the one holding the pools
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
        geom[lane] = QueryGeom{base, off + incl - nt, nt, ng, nn, tok0, pb, pe, rank, 0};
    }
    lds_barrier();
    const int total = (int)(geom[63].first + geom[63].ntiles);
    int tile = blockIdx.x;
    for (; tile < total; tile += gridDim.x) {
        int t, j;
        if (AD != 0 && tile < (int)uniform32((int)geom[0].first)) {
            t = __ffsll((long long)__ballot(geom[lane].rank == tile)) - 1;   // the tile-th query's last tile
            j = (uniform32(geom[t].ng) - 1) >> 2;
        } else {
            // query of the tile: the number of queries whose tiles all come before it
            t = __popcll(__ballot(geom[lane].first + geom[lane].ntiles <= (uint32_t)tile));
            j = tile - uniform32((int)geom[t].first);
        }
        const int grp = 4 * j + wave;
        const bool has = grp < uniform32(geom[t].ng);
        const int n_vis = uniform32(geom[t].nn);
        const int p0 = grp * kGroupPools;
        // The tile's A operand: wave w loads heads 8 w .. 8 w + 7 (two 16-byte
        // pieces per lane), plus the head weights; issued before the pool rows.
        // (Buffer loads: the lane part of each address is a 32-bit offset.)
        u32x4 qv[2];
        {
            const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q_idx + (int64_t)t * (kHI * kDI), kHI * kDI * 2);
            const uint32_t loff = (uint32_t)((lane >> 4) * (kDI * 2) + (lane & 15) * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)              // piece lane + 64 i: head 8 w + 4 i + lane / 16, dims 8 (lane % 16) ..
                qv[i] = ld_buf128(rq, loff, (uint32_t)((8 * wave + 4 * i) * (kDI * 2)));
        }
        const float wt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            buffer_rsrc(w + (int64_t)t * kHI, kHI * 4), (uint32_t)min(lane, 7) * 4u, (uint32_t)(32 * wave), 0));
        // A wave past the query's last group re-reads the tile's first row
        // (unconditional loads keep the wait counts exact).
        u32x4 v[I8 ? 8 : 16];
        float psc = 0.f;                               // INT8: the scale of pool p0 + lane
        const int lp0 = has ? p0 : p0 - kGroupPools * wave;
        {
            const int64_t gb = (int64_t)uniform64((uint64_t)geom[t].base);
            const int64_t row0 = PAGED ? pm.block((int)gb, lp0 / kPagePools) * kPagePools : gb + lp0;
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
        __builtin_amdgcn_sched_barrier(0);             // every load in flight before the A operand is shared
        // the group list length, while the rows are in flight
        const int gm = CANDS && n_vis > select_k ? group_quota<!LONG>(select_k, n_vis) : 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = lane + 64 * i;
            *reinterpret_cast<u32x4*>(&s_q[(8 * wave + (k >> 4)) * kQStride + 8 * (k & 15)]) = qv[i];
        }
        if (lane < 8) s_w[8 * wave + lane] = wt;
        lds_barrier();
        if (has) {
            // A completed pool's row, built with the pool tasks' code, into s_new[wave].
            auto build = [&](const PoolRaw128& r) {
                PoolIn<kDI, uint16_t> in;
                pool_raw_in(r, in);
                uint16_t ov[2];
                pool_values<kDI, uint16_t>(in, ap.ln_w, ap.ln_b, ap.eps, ov);
                s_new[AD ? wave : 0][lane] = (uint32_t)ov[0] | ((uint32_t)ov[1] << 16);
                wave_lds_fence();
            };
            float s;
            if constexpr (I8) {
                IdxQueryI8 Q;
                load_idx_query_lds_i8(s_q, kQStride, s_w, Q);
                s = score_pool_group_i8(Q, v, psc);
            } else {
                IdxQuery Q;
                load_idx_query_lds(s_q, kQStride, s_w, Q);
                s = score_pool_group(Q, v);
            }
            if constexpr (AD != 0 && I8) {
                // Rebuilt pools in the INT8 form: the pool tasks' values and
                // quantiser, the codes through s_new[wave] as 128 bytes.
                const int nb = max(uniform32(geom[t].pb), p0);
                const int ne = min(min(uniform32(geom[t].pe), p0 + kGroupPools), n_vis);
                const int64_t tok0 = (int64_t)uniform64((uint64_t)geom[t].tok0);
                for (int pp = nb; pp < ne; ++pp) {
                    PoolRaw128 r;
                    pool_raw_load(ap.k, ap.gate, tok0 + 4 * (int64_t)pp, r);
                    PoolIn<kDI, uint16_t> in;
                    pool_raw_in(r, in);
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
                    IdxQueryI8 Q2;                     // reloaded: Q is not kept through the rebuild
                    load_idx_query_lds_i8(s_q, kQStride, s_w, Q2);
                    const float s2 = score_pool_column_i8(Q2, w0, w1, sc);
                    if (lane == pp - p0) s = s2;
                    wave_lds_fence();                  // s_new is rewritten by the next pool
                }
            } else if constexpr (AD != 0) {
                // Score each rebuilt pool (score_pool_column: lane pp - p0 gets
                // the bits the group's own scoring would have given it).
                const int nb = max(uniform32(geom[t].pb), p0);
                const int ne = min(min(uniform32(geom[t].pe), p0 + kGroupPools), n_vis);
                const int64_t tok0 = (int64_t)uniform64((uint64_t)geom[t].tok0);
                for (int pp = nb; pp < ne; ++pp) {
                    PoolRaw128 r;
                    pool_raw_load(ap.k, ap.gate, tok0 + 4 * (int64_t)pp, r);
                    build(r);
                    const int g = lane >> 4;
                    u32x4 nb4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) nb4[i] = *reinterpret_cast<const u32x4*>(&s_new[wave][16 * i + 4 * g]);
                    IdxQuery Q2;                       // reloaded: Q is not kept through the rebuild
                    load_idx_query_lds(s_q, kQStride, s_w, Q2);
                    const float s2 = score_pool_column(Q2, nb4);
                    if (lane == pp - p0) s = s2;
                    wave_lds_fence();                  // s_new is rewritten by the next pool
                }
            }
            const int p = p0 + lane;
            {
                // a buffer store: pools at or past the row stride fall outside its range
                const __amdgpu_buffer_rsrc_t rs =
                    buffer_rsrc(scores + (int64_t)t * stride + p0, (uint32_t)(min(stride - p0, kGroupPools) * 4));
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p < n_vis ? s : -INFINITY), rs,
                                                      (uint32_t)lane * 4u, 0, 0);
            }
            if constexpr (CANDS) {
                if (n_vis > select_k) {
                    if (LONG && n_vis > kShortListPools)
                        keep_group_best(s, p < n_vis, p, 0, gm, s_long + wave * gm, s_long_n + wave,
                                        [](uint64_t* q, uint64_t x) { *q = x; },
                                        [](int32_t* q, uint32_t x) { *q = (int32_t)x; });
                    else
                        keep_group_best(s, p < n_vis, p, grp, gm,
                                        cand + (int64_t)t * kGroupCandCap, cand_n + (int64_t)t * kMaxGroups,
                                        [](uint64_t* q, uint64_t x) { *q = x; },
                                        [](int32_t* q, uint32_t x) { *q = (int32_t)x; });
                }
            }
        }
        if constexpr (CANDS && LONG) {
            if (n_vis > kShortListPools && n_vis > select_k) {   // the same for the whole workgroup
                lds_barrier();
                if (wave == 0) {
                    // lane l: entry l % gm of wave l / gm's list (lane order is id
                    // order); a wave past the query's last group kept nothing
                    const int wv = lane / gm;
                    const uint64_t e = lane < 4 * gm ? s_long[lane] : 0ull;
                    const bool ok = lane < 4 * gm && 4 * j + wv < uniform32(geom[t].ng);
                    keep_best_keys(ok ? (uint32_t)(e >> 32) : 0u, ok && (e >> 32) != 0ull, 0xFFFFFFFFu - (uint32_t)e,
                                   min(max(n_vis - kLongGroupPools * j, 0), kLongGroupPools), j, gm,
                                   cand + (int64_t)t * kGroupCandCap, cand_n + (int64_t)t * kMaxGroups,
                                   [](uint64_t* q, uint64_t x) { *q = x; },
                                   [](int32_t* q, uint32_t x) { *q = (int32_t)x; });
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
        const int from = geom[t].ng * kGroupPools;
        float* out = scores + (int64_t)t * stride;
        for (int p = from + gw * kGroupPools + lane; p < stride; p += W * kGroupPools) out[p] = -INFINITY;
    }
}

// Vector kernel for other geometries (tiny configurations): one thread per
// (query, pool), fp32 dot products over bf16 inputs.
__global__ __launch_bounds__(256) void k_scores_generic(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ pools, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int HI, int DI, int stride, float* __restrict__ scores) {
    const int t = blockIdx.y;
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= stride) return;
    const int b = q_seq[t];
    const int f = first_valid[b];
    const int qp = q_pos[t];
    const int n_vis = qp >= f ? (qp - f + 1) >> 2 : 0;
    float* out = scores + (int64_t)t * stride;
    if (p >= n_vis) {
        out[p] = -INFINITY;
        return;
    }
    const uint16_t* pr = pools + (pool_base[b] + p) * DI;
    const uint16_t* qr = q_idx + (int64_t)t * HI * DI;
    float s = 0.f;
    for (int h = 0; h < HI; ++h) {
        float dot = 0.f;
        for (int c = 0; c < DI; ++c) dot += bf16_to_f32(qr[h * DI + c]) * bf16_to_f32(pr[c]);
        s += w[(int64_t)t * HI + h] * fmaxf(dot, 0.f);
    }
    out[p] = s;
}

}  // namespace dsa

namespace dsa_host {

// Events the next scoring launch (k_scores_groups or k_scores_mfma, from any
// entry point) records around the kernel itself; one-shot.
namespace {
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;
}  // namespace

void take_events(hipEvent_t& a, hipEvent_t& b) {
    a = t_ev_start;
    b = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
}

void time_next_scoring_launch(hipEvent_t start, hipEvent_t stop) {
    t_ev_start = start;
    t_ev_stop = stop;
}

// Prefill scoring geometry (k_scores_mfma): waves per workgroup, queries per workgroup.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillQPB = 24;

// Workgroups (one 256-pool tile each) for k_scores_groups: every tile of
// every query if that fits, else 4 per CU, which stay resident.
static unsigned scores_groups_grid(int32_t T, int32_t stride) {
    const int64_t wgs = cdiv(cdiv(stride, dsa::kGroupPools), 4) * (int64_t)T;
    return (unsigned)std::min<int64_t>(wgs, 4 * (int64_t)device_info().cu_count);
}

hipError_t launch_index_scores(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                               const uint16_t* pools, const dsa_seqs& seqs, int32_t num_seqs,
                               const int32_t* q_seq,
                               const int32_t* q_pos, int32_t T, int32_t stride, float* scores,
                               hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    if (d.idx_heads == dsa::kHI && d.idx_dim == dsa::kDI) {
        if (T <= dsa::kDecMaxT) {
            // Decode: one wave per 64-pool group, a resident grid.
            hipEvent_t ev0, ev1;
            take_events(ev0, ev1);
            hipExtLaunchKernelGGL((dsa::k_scores_groups<false, 0>), dim3(scores_groups_grid(T, stride)), dim3(256), 0,
                                  s, ev0, ev1, 0, q_idx, w, pools, seqs.first_valid, seqs.pool_base, q_seq,
                                  q_pos, T, num_seqs, stride, scores, 0, nullptr, nullptr, dsa::AppendArgs{}, nullptr, dsa::PagedMap{});
        } else {
            // Prefill: 256 resident pools per workgroup (4 waves), 24 queries
            // per workgroup: three workgroups per CU (168 VGPRs) and about 2,900
            // workgroups per 512-query chunk of the prefill config (3.8 rounds of
            // 768), where 8-wave workgroups of 64 queries ran one per CU in 2.06
            // rounds (242 us a chunk against 169 us; 32 or 48 queries: 173, 171).
            dim3 grid((unsigned)cdiv(stride, kPrefillWaves * 64), (unsigned)cdiv(T, kPrefillQPB)),
                block(kPrefillWaves * 64);
            hipEvent_t ev0, ev1;
            take_events(ev0, ev1);
            hipExtLaunchKernelGGL((dsa::k_scores_mfma<kPrefillWaves, 2>), grid, block, 0, s, ev0, ev1, 0, q_idx, w,
                                  pools, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, kPrefillQPB, stride,
                                  scores, 0, nullptr, nullptr);
        }
    } else {
        dim3 grid((unsigned)cdiv(stride, 256), (unsigned)T), block(256);
        hipLaunchKernelGGL(dsa::k_scores_generic, grid, block, 0, s, q_idx, w, pools,
                           seqs.first_valid, seqs.pool_base, q_seq, q_pos, d.idx_heads, d.idx_dim,
                           stride, scores);
    }
    return hipGetLastError();
}

// Scores and group lists for any number of queries: the decode kernel for
// at most 64, the prefill kernel (with its group lists) for more.
hipError_t launch_scores_lists(const dsa_dims& d, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                               const dsa_seqs& seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                               int32_t T, int32_t stride, float* scores, void* ws, hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    if (T <= dsa::kDecMaxT)
        return launch_scores_with_groups(d, q_idx, w, pools, seqs, num_seqs, q_seq, q_pos, T, stride, scores, ws, s);
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    dim3 grid((unsigned)cdiv(stride, kPrefillWaves * 64), (unsigned)cdiv(T, kPrefillQPB)), block(kPrefillWaves * 64);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
    hipExtLaunchKernelGGL((dsa::k_scores_mfma<kPrefillWaves, 2, true>), grid, block, 0, s, ev0, ev1, 0, q_idx, w,
                          pools, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, kPrefillQPB, stride, scores,
                          d.index_topk / d.kpool, cand, cand_n);
    return hipGetLastError();
}

bool scores_select_grouped(const dsa_dims& d, int32_t T, int32_t stride) {
    return d.idx_heads == dsa::kHI && d.idx_dim == dsa::kDI && T <= dsa::kDecMaxT && d.kpool == 4 &&
           stride <= dsa::kListMaxPools && d.index_topk / d.kpool <= dsa::kGroupMaxK;
}

bool scores_lists_short(const dsa_dims& d, int32_t T, int32_t stride) {
    return scores_select_grouped(d, T, stride) && stride <= dsa::kShortListPools;
}

size_t scores_select_group_bytes(int32_t T) {
    return ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256 + ((size_t)T * dsa::kMaxGroups * 4 + 255) / 256 * 256;
}

hipError_t launch_scores_with_groups(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                     const uint16_t* pools, const dsa_seqs& seqs, int32_t num_seqs,
                                     const int32_t* q_seq,
                                     const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                     hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
#define DSA_SCORES_GROUPS(LONG)                                                                                    \
    hipExtLaunchKernelGGL((dsa::k_scores_groups<true, 0, false, false, LONG>), dim3(scores_groups_grid(T, stride)),  \
                          dim3(256), 0, s, ev0, ev1, 0, q_idx, w, pools, seqs.first_valid, seqs.pool_base, q_seq,    \
                          q_pos, T, num_seqs, stride, scores, d.index_topk / d.kpool, cand, cand_n,                  \
                          dsa::AppendArgs{}, nullptr, dsa::PagedMap{})
    if (stride > dsa::kShortListPools) DSA_SCORES_GROUPS(true);
    else DSA_SCORES_GROUPS(false);
#undef DSA_SCORES_GROUPS
    return hipGetLastError();
}


bool append_scores_fused(const dsa_dims& d, int dtype) {
    return dtype == DSA_BF16 && d.idx_dim == dsa::kDI &&
           (d.latent_dim == 64 || d.latent_dim == 128 || d.latent_dim == 256 || d.latent_dim == 512);
}


hipError_t launch_append_scores_groups(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                       const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                       const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                       const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                       uint16_t* pools, const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                       const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                       hipStream_t s) {
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    dsa::AppendArgs ap;
    if (!make_append_args(d, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, seqs, num_seqs, pool_begin, pool_end,
                          max_pools, pools, nullptr, ap))
        return hipErrorInvalidValue;
    const unsigned grid = fused_grid(T, stride, ap.tasks);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
#define DSA_APPEND_SCORES(D, LONG)                                                                                  \
    hipExtLaunchKernelGGL((dsa::k_scores_groups<true, D, false, false, LONG>), dim3(grid), dim3(256), 0, s, ev0, ev1, \
                          0, q_idx, w, pools, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, num_seqs, stride,  \
                          scores, d.index_topk / d.kpool, cand, cand_n, ap, nullptr, dsa::PagedMap{})
    if (stride > dsa::kShortListPools) {
        switch (d.latent_dim) {
            case 512: DSA_APPEND_SCORES(512, true); break;
            case 256: DSA_APPEND_SCORES(256, true); break;
            case 128: DSA_APPEND_SCORES(128, true); break;
            default: DSA_APPEND_SCORES(64, true); break;
        }
    } else {
        switch (d.latent_dim) {
            case 512: DSA_APPEND_SCORES(512, false); break;
            case 256: DSA_APPEND_SCORES(256, false); break;
            case 128: DSA_APPEND_SCORES(128, false); break;
            default: DSA_APPEND_SCORES(64, false); break;
        }
    }
#undef DSA_APPEND_SCORES
    return hipGetLastError();
}

// ------------------------------------------------------------------ paged pools

hipError_t launch_scores_with_groups_paged(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                           const uint16_t* pools, const int32_t* first_valid, const int32_t* table,
                                           int32_t table_stride, int32_t num_seqs, const int32_t* q_seq,
                                           const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                           hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
    hipExtLaunchKernelGGL((dsa::k_scores_groups<true, 0, false, true>), dim3(scores_groups_grid(T, stride)), dim3(256),
                          0, s, ev0, ev1, 0, q_idx, w, pools, first_valid, nullptr, q_seq, q_pos, T, num_seqs, stride,
                          scores, d.index_topk / d.kpool, cand, cand_n, dsa::AppendArgs{}, nullptr,
                          dsa::PagedMap{table, table_stride});
    return hipGetLastError();
}

// ------------------------------------------------------------------ INT8 pools

hipError_t launch_index_scores_int8(const dsa_dims& d, const uint16_t* q_idx, const float* w, const int8_t* codes,
                                    const float* scales, const dsa_seqs& seqs, int32_t num_seqs, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t T, int32_t stride, float* scores, hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
    hipExtLaunchKernelGGL((dsa::k_scores_groups<false, 0, true>), dim3(scores_groups_grid(T, stride)), dim3(256), 0, s,
                          ev0, ev1, 0, q_idx, w, codes, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T,
                          num_seqs, stride, scores, 0, nullptr, nullptr, dsa::AppendArgs{},
                          const_cast<float*>(scales), dsa::PagedMap{});
    return hipGetLastError();
}

hipError_t launch_scores_with_groups_int8(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                          const int8_t* codes, const float* scales, const dsa_seqs& seqs,
                                          int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                          int32_t stride, float* scores, void* ws, hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
#define DSA_SCORES_GROUPS8(LONG)                                                                                   \
    hipExtLaunchKernelGGL((dsa::k_scores_groups<true, 0, true, false, LONG>), dim3(scores_groups_grid(T, stride)),   \
                          dim3(256), 0, s, ev0, ev1, 0, q_idx, w, codes, seqs.first_valid, seqs.pool_base, q_seq,    \
                          q_pos, T, num_seqs, stride, scores, d.index_topk / d.kpool, cand, cand_n,                  \
                          dsa::AppendArgs{}, const_cast<float*>(scales), dsa::PagedMap{})
    if (stride > dsa::kShortListPools) DSA_SCORES_GROUPS8(true);
    else DSA_SCORES_GROUPS8(false);
#undef DSA_SCORES_GROUPS8
    return hipGetLastError();
}

hipError_t launch_append_scores_groups_int8(const dsa_dims& d, const void* latent, int64_t n, int64_t ld,
                                            const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                            const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                                            int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                                            int32_t max_pools, int8_t* codes, float* scales, const uint16_t* q_idx,
                                            const float* w, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                            int32_t stride, float* scores, void* ws, hipStream_t s) {
    uint64_t* cand;
    int32_t* cand_n;
    group_lists(ws, T, cand, cand_n);
    dsa::AppendArgs ap;
    if (!make_append_args(d, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, seqs, num_seqs, pool_begin, pool_end,
                          max_pools, nullptr, codes, ap))
        return hipErrorInvalidValue;
    const unsigned grid = fused_grid(T, stride, ap.tasks);
    hipEvent_t ev0, ev1;
    take_events(ev0, ev1);
#define DSA_APPEND_SCORES8(D, LONG)                                                                                 \
    hipExtLaunchKernelGGL((dsa::k_scores_groups<true, D, true, false, LONG>), dim3(grid), dim3(256), 0, s, ev0, ev1,  \
                          0, q_idx, w, codes, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, num_seqs, stride,  \
                          scores, d.index_topk / d.kpool, cand, cand_n, ap, scales, dsa::PagedMap{})
    if (stride > dsa::kShortListPools) {
        switch (d.latent_dim) {
            case 512: DSA_APPEND_SCORES8(512, true); break;
            case 256: DSA_APPEND_SCORES8(256, true); break;
            case 128: DSA_APPEND_SCORES8(128, true); break;
            default: DSA_APPEND_SCORES8(64, true); break;
        }
    } else {
        switch (d.latent_dim) {
            case 512: DSA_APPEND_SCORES8(512, false); break;
            case 256: DSA_APPEND_SCORES8(256, false); break;
            case 128: DSA_APPEND_SCORES8(128, false); break;
            default: DSA_APPEND_SCORES8(64, false); break;
        }
    }
#undef DSA_APPEND_SCORES8
    return hipGetLastError();
}

}  // namespace dsa_host
