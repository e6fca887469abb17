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
#include "dsa_common.h"
#include "dsa_launch.h"
#include "topk_core.h"

namespace dsa {

constexpr int kHI = 32, kDI = 128, kQROW = kDI + 8;   // padded LDS row (bf16 elements)
constexpr int kQBYTES = kHI * kDI * 2;                // 8 KB per query

template <int WAVES, int QB>
__global__ __launch_bounds__(WAVES * 64) void k_scores_mfma(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ pools, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int T, int q_per_block, int stride,
    float* __restrict__ scores) {
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
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + j * 8));
                acc0 = mfma32(a, as_bf16x8(breg[0][j]), acc0);
                acc1 = mfma32(a, as_bf16x8(breg[1][j]), acc1);
            }
            // Heads held by this lane: 8*(r/4) + 4*g + (r%4).
            const float* wq = &w_lds[qi][4 * g];
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float wh = wq[8 * (r >> 2) + (r & 3)];
                s0 += wh * fmaxf(acc0[r], 0.f);
                s1 += wh * fmaxf(acc1[r], 0.f);
            }
            s0 += __shfl_xor(s0, 32, 64);
            s1 += __shfl_xor(s1, 32, 64);
            const float sv = g == 0 ? s0 : s1;
            const int p = p0 + g * 32 + n;                 // lanes 0-31: tile 0, 32-63: tile 1
            if (p < stride) out[p] = p < n_vis ? sv : -INFINITY;
        }
    }
}

// Decode kernel (persistent).  Work is a flat list of 256-pool tiles over all
// queries (a query with n_vis pools has ceil(n_vis / 256) tiles), so ragged
// lengths balance across the grid; each workgroup (4 waves) walks tiles
// blockIdx.x, blockIdx.x + gridDim.x, ...  A tile (64 KB, contiguous in HBM)
// is fetched with fully coalesced 16-byte loads -- consecutive lanes read
// consecutive chunks, so each load instruction covers whole cache lines --
// into registers one tile ahead (with the next query's A operand and head
// weights), then stored to LDS with an XOR swizzle (chunk c of pool row r goes
// to slot c ^ (r & 15)) so that the MFMA B-operand reads hit all 64 banks
// once.  Each wave runs two 32-pool N-tiles of the tile.  Pools past a
// query's visible count are written as -inf, by the partial tile and by a
// final fill of [tiles*256, stride).
// With CANDS, each wave also keeps its 64-pool group's best m pools for the
// selection (keep_group_best), for queries with more visible pools than
// select_k.
constexpr int kDecTile = 256;
constexpr int kDecMaxT = 64;
template <bool CANDS>
__global__ __launch_bounds__(256) void k_scores_decode(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ pools, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int T, int stride, float* __restrict__ scores,
    int select_k, uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n) {
    __shared__ u32x4 tile[kDecTile * 16];
    __shared__ int s_first[kDecMaxT + 1];     // first flat tile of each query
    __shared__ int s_nvis[kDecMaxT];
    __shared__ int64_t s_base[kDecMaxT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, g = lane >> 5;

    if (tid < 64) {
        int nt = 0;
        if (tid < T) {
            const int b = q_seq[tid];
            const int f = first_valid[b];
            const int qp = q_pos[tid];
            const int nv = qp >= f ? (qp - f + 1) >> 2 : 0;
            s_nvis[tid] = nv;
            s_base[tid] = pool_base[b];
            nt = (min(nv, stride) + kDecTile - 1) / kDecTile;
        }
        int x = nt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (tid < T) s_first[tid] = x - nt;
        if (tid == 63) s_first[kDecMaxT] = x;
    }
    lds_barrier();
    const int total = s_first[kDecMaxT];

    auto locate = [&](int i, int& t, int& p0) {
        int q = 0;
        while (q + 1 < T && s_first[q + 1] <= i) ++q;
        t = q;
        p0 = (i - s_first[q]) * kDecTile;
    };
    u32x4 v[16];
    u32x4 anext[8];
    f32x4 wnext[4];
    auto prefetch = [&](int i) {
        int t, p0;
        locate(i, t, p0);
        const int lim = min(s_nvis[t] - p0, kDecTile);
        const u32x4* src = reinterpret_cast<const u32x4*>(pools + (s_base[t] + p0) * kDI);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int id = tid + k * 256;                    // row id >> 4, chunk id & 15
            v[k] = (id >> 4) < lim ? src[id] : u32x4{0u, 0u, 0u, 0u};
        }
        // A operand: head n, k = g*64 + j*8 + e (chunk g*8 + j).  D rows: 8*(r/4) + 4*g + (r%4).
        const uint16_t* qrow = q_idx + ((int64_t)t * kHI + n) * kDI + g * 64;
#pragma unroll
        for (int j = 0; j < 8; ++j) anext[j] = *reinterpret_cast<const u32x4*>(qrow + j * 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) wnext[k] = *reinterpret_cast<const f32x4*>(w + (int64_t)t * kHI + 8 * k + 4 * g);
    };

    int i = blockIdx.x;
    if (i < total) prefetch(i);
    for (; i < total; i += gridDim.x) {
        int t, p0;
        locate(i, t, p0);
        const int n_vis = s_nvis[t];
        u32x4 areg[8];
        f32x4 wv[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) areg[j] = anext[j];
#pragma unroll
        for (int k = 0; k < 4; ++k) wv[k] = wnext[k];
        lds_barrier();                                     // previous tile's LDS readers are done
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int id = tid + k * 256;
            const int row = id >> 4;
            tile[row * 16 + ((id & 15) ^ (row & 15))] = v[k];
        }
        if (i + (int)gridDim.x < total) prefetch(i + gridDim.x);
        lds_barrier();
        float sc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int row = wave * 64 + nt * 32 + n;
            f32x16 acc = {};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc = mfma32(as_bf16x8(areg[j]), as_bf16x8(tile[row * 16 + ((g * 8 + j) ^ (row & 15))]), acc);
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) s += wv[r >> 2][r & 3] * fmaxf(acc[r], 0.f);
            sc[nt] = s + __shfl_xor(s, 32, 64);
        }
        const int p = p0 + wave * 64 + g * 32 + n;            // lanes 0-31: N-tile 0, 32-63: N-tile 1
        if (p < stride) scores[(int64_t)t * stride + p] = p < n_vis ? sc[g] : -INFINITY;
        if constexpr (CANDS) {
            const int nn = min(n_vis, stride);
            if (nn > select_k)                                  // lane order is id order
                keep_group_best(sc[g], p < nn, p, p / kGroupPools, group_quota(select_k, nn),
                                cand + (int64_t)t * kGroupCandCap, cand_n + (int64_t)t * kMaxGroups,
                                [](uint64_t* q, uint64_t v) { *q = v; }, [](int32_t* q, uint32_t v) { *q = (int32_t)v; });
        }
    }
    // Pools past the last visible tile of each query.
    for (int t = 0; t < T; ++t) {
        const int from = (s_first[t + 1 < T ? t + 1 : kDecMaxT] - s_first[t]) * kDecTile;
        float* out = scores + (int64_t)t * stride;
        for (int p = from + blockIdx.x * 256 + tid; p < stride; p += gridDim.x * 256) out[p] = -INFINITY;
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

hipError_t launch_index_scores(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                               const uint16_t* pools, const dsa_seqs& seqs, const int32_t* q_seq,
                               const int32_t* q_pos, int32_t T, int32_t stride, float* scores,
                               hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    if (d.idx_heads == dsa::kHI && d.idx_dim == dsa::kDI) {
        if (T <= 64) {
            // Decode: persistent, two 64 KB-LDS workgroups per CU over a flat tile list.
            const int64_t tiles = cdiv(stride, dsa::kDecTile) * (int64_t)T;
            const int grid = (int)std::min<int64_t>(tiles, 2 * (int64_t)device_info().cu_count);
            hipLaunchKernelGGL((dsa::k_scores_decode<false>), dim3((unsigned)grid), dim3(256), 0, s, q_idx, w,
                               pools, seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, stride, scores, 0,
                               nullptr, nullptr);
        } else {
            // Prefill: 512 resident pools per workgroup, 64 queries per workgroup.
            const int qpb = 64;
            dim3 grid((unsigned)cdiv(stride, 512), (unsigned)cdiv(T, qpb)), block(512);
            hipLaunchKernelGGL((dsa::k_scores_mfma<8, 4>), grid, block, 0, s, q_idx, w, pools,
                               seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, qpb, stride, scores);
        }
    } else {
        dim3 grid((unsigned)cdiv(stride, 256), (unsigned)T), block(256);
        hipLaunchKernelGGL(dsa::k_scores_generic, grid, block, 0, s, q_idx, w, pools,
                           seqs.first_valid, seqs.pool_base, q_seq, q_pos, d.idx_heads, d.idx_dim,
                           stride, scores);
    }
    return hipGetLastError();
}

bool scores_select_grouped(const dsa_dims& d, int32_t T, int32_t stride) {
    return d.idx_heads == dsa::kHI && d.idx_dim == dsa::kDI && T <= dsa::kDecMaxT && d.kpool == 4 &&
           stride <= dsa::kMaxGroups * dsa::kGroupPools && d.index_topk / d.kpool <= dsa::kGroupMaxK;
}

size_t scores_select_group_bytes(int32_t T) {
    return ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256 + ((size_t)T * dsa::kMaxGroups * 4 + 255) / 256 * 256;
}

hipError_t launch_scores_with_groups(const dsa_dims& d, const uint16_t* q_idx, const float* w,
                                     const uint16_t* pools, const dsa_seqs& seqs, const int32_t* q_seq,
                                     const int32_t* q_pos, int32_t T, int32_t stride, float* scores, void* ws,
                                     hipStream_t s) {
    if (T == 0 || stride == 0) return hipSuccess;
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
    int32_t* cand_n = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                                 ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256);
    const int64_t tiles = cdiv(stride, dsa::kDecTile) * (int64_t)T;
    const int grid = (int)std::min<int64_t>(tiles, 2 * (int64_t)device_info().cu_count);
    hipLaunchKernelGGL((dsa::k_scores_decode<true>), dim3((unsigned)grid), dim3(256), 0, s, q_idx, w, pools,
                       seqs.first_valid, seqs.pool_base, q_seq, q_pos, T, stride, scores, d.index_topk / d.kpool,
                       cand, cand_n);
    return hipGetLastError();
}

}  // namespace dsa_host
