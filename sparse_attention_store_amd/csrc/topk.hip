// topk_select: per query, the K = min(select_k, n_vis) best pools by
// (score descending, pool id ascending), emitted in ascending id order and
// padded with -1 ([Ref] Functions: topk_pools; [Flash] Stream C:
// indexer_topk512).  Optionally the same launches also write the expanded
// index list ([Ref] Functions: expand_selection).
//
// The order is total on the 64-bit composite (key << 32 | ~id), key being the
// order-preserving uint32 image of the fp32 score (-0 mapped to +0).
//  A. Tiles of 256 pools: one workgroup per tile sorts the tile's composites
//     (bitonic, in registers and LDS) and keeps its best m, m sized from the
//     row's tile count so that m is at least 2.5 times a tile's mean share of
//     the K (>= 16, a power of two).  The kept ones are written in ascending
//     id order, with a flag saying whether the tile had more pools than m.
//  B. One 1024-thread workgroup per row selects the best K of the union of
//     the tile lists (held in registers; the lists are in ascending id order,
//     so the 32-bit key selection with ties taken in list order applies the
//     tie rule).  The union holds the answer unless some tile that dropped
//     pools had all m of its kept ones selected -- then a dropped one might
//     belong too.  The workgroup checks exactly that and, if it happens,
//     selects again from the row's scores with an exact streaming radix
//     select, so the result never depends on the score distribution.
// Rows of at most kDirectPools pools skip A and B: one 1024-thread workgroup
// per row holds the row's keys in registers (KPT consecutive pools per thread,
// so slot order is id order) and selects the best K of them directly
// (k_topk_direct).
// The K-th largest key is found by range bucketing in LDS: each pass
// histograms the keys inside [lo, hi] into one bucket per thread, of width
// 2^sh (the key offset shifted right), keeps the bucket that holds rank K and
// narrows [lo, hi] to it, until that bucket is taken whole or one key value is
// left, whose first `need` occurrences in id order are taken.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "topk_core.h"
#include "group_select.h"

namespace dsa {

constexpr int kTile = 256;                  // pools per stage-A workgroup
constexpr int kBNT = 1024;
constexpr int kMaxK = 1024;                 // select_k limit
constexpr int kMaxTiles = 1024;             // 262,144 pools per row
constexpr int kMaxKpt = 16;                 // stage-B slots per thread
constexpr int kDirectKpt = 40;              // k_topk_direct: keys per thread
constexpr int kDirectPools = kDirectKpt * kBNT;   // 40,960 pools per row
constexpr int kIncomplete = 1 << 30;        // tile count flag: the tile dropped pools

// Kept per tile for a row of `ntiles` tiles.
__host__ __device__ inline int tile_quota(int select_k, int ntiles) {
    const int want = (5 * select_k + 2 * ntiles - 1) / (2 * ntiles);
    int m = 16;
    while (m < want && m < kTile) m <<= 1;
    return m;
}

// Candidate slots per row: ntiles * tile_quota(ntiles) <= 16 ntiles + 5 K + 256
// for every ntiles (m = 16; or m < 2 ceil(2.5 K / ntiles); or m = 256 only
// when ntiles < 5 K / 256), rounded up to even so that every row starts on
// 16 bytes for stage B's paired-slot loads.
__host__ __device__ inline int64_t cand_row_cap(int select_k, int ntiles_max) {
    return (16LL * ntiles_max + 5LL * select_k + 257) & ~1LL;
}

// Slots stage B reads for the longest row: max over ntiles <= ntiles_max of
// ntiles * tile_quota(ntiles), at most max(16 ntiles_max, 5 K + 2 ntiles_max),
// which is 16,384 = kMaxKpt * kBNT at kMaxK and kMaxTiles.
inline int64_t max_row_slots(int select_k, int ntiles_max) {
    int64_t slots = 0;
    for (int n = 1; n <= ntiles_max; ++n) slots = std::max<int64_t>(slots, (int64_t)n * tile_quota(select_k, n));
    return slots;
}


// ---------------------------------------------------------------- stage A

__global__ __launch_bounds__(kTile) void k_topk_tiles(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int select_k, int64_t cap,
    int ntiles_max, uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n) {
    __shared__ uint64_t xs[2][kTile];
    __shared__ uint32_t wcount[kTile / 64];
    __shared__ uint64_t theta_sh;
    const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int n = min(n_vis, stride);
    if (n <= select_k) return;                               // stage B selects every pool
    const int ntiles = (n + kTile - 1) / kTile;
    if (c >= ntiles) return;
    const int m = tile_quota(select_k, ntiles);
    const int id = c * kTile + tid;
    const bool valid = id < n;
    const uint64_t comp = valid ? ((uint64_t)f32_key(scores[(int64_t)t * stride + id]) << 32) |
                                      (uint64_t)(0xFFFFFFFFu - (uint32_t)id)
                                : 0ull;
    const int nvalid = min(n - c * kTile, kTile);
    uint64_t theta = 1ull;                                   // keep composites >= theta
    if (nvalid > m) {
        // Bitonic sort, descending; lanes exchange by shuffles, waves through LDS.
        uint64_t v = comp;
        int buf = 0;
#pragma unroll
        for (int k = 2; k <= kTile; k <<= 1)
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1) {
                uint64_t o;
                if (j < 64) {
                    o = shfl_xor_k(v, j);
                } else {
                    xs[buf][tid] = v;
                    lds_barrier();
                    o = xs[buf][tid ^ j];
                    buf ^= 1;
                }
                const bool desc = (tid & k) == 0, lower = (tid & j) == 0;
                v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
            }
        if (tid == m - 1) theta_sh = v;
        lds_barrier();
        theta = theta_sh;
    }
    const bool pick = comp >= theta;                         // comp 0 (absent) never passes
    const uint64_t bal = __ballot(pick);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    const int w = tid >> 6;
    if ((tid & 63) == 0) wcount[w] = (uint32_t)__popcll(bal);
    lds_barrier();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kTile / 64; ++i) {
        base += i < w ? wcount[i] : 0u;
        total += wcount[i];
    }
    if (pick) cand[(int64_t)t * cap + (int64_t)c * m + base + below] = comp;
    if (tid == 0) cand_n[(int64_t)t * ntiles_max + c] = (int32_t)total | (nvalid > m ? kIncomplete : 0);
}

// ---------------------------------------------------------------- stage B

template <int KPT>
__global__ __launch_bounds__(kBNT) void k_topk_rows(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int stride, int select_k,
    int64_t cap, int ntiles_max, const uint64_t* __restrict__ cand, const int32_t* __restrict__ cand_n, Emit e) {
    __shared__ TopSelShared<kBNT, KPT> T;
    __shared__ int32_t sel[kMaxK];
    __shared__ uint32_t tpicked[kMaxTiles];
    __shared__ int fail;
    const int t = blockIdx.x, tid = threadIdx.x;
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int n = min(n_vis, stride);
    if (n <= select_k) {                                     // every visible pool is selected
        emit_selection<kBNT>(nullptr, n, select_k, t, b, f, qp, n_vis, e);
        return;
    }
    const int ntiles = (n + kTile - 1) / kTile;
    const int m = tile_quota(select_k, ntiles);
    const int msh = __ffs(m) - 1;
    const int M = ntiles * m;                                // slots: tile c at [c*m, c*m + count_c)
    const int32_t* cn = cand_n + (int64_t)t * ntiles_max;
    const uint64_t* cr = cand + (int64_t)t * cap;
    if (tid < kMaxTiles) tpicked[tid] = 0u;
    if (tid == 0) fail = 0;
    const int s0 = tid * KPT;
    uint32_t key[KPT];                                       // a pool's id is re-read once it is picked
    {
        // Every load at once: this thread's slots (two per 16-byte load) and
        // the counts of the (at most two, m >= 16) tiles they lie in, through
        // descriptors bounded to the row's M slots and ntiles counts (reads
        // past them give 0), so no load waits on another and none branches.
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(cr, (uint32_t)M * 8u);
        const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(cn, (uint32_t)ntiles * 4u);
        const int tile0 = s0 >> msh;
        const uint32_t cnt0 = __builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)tile0 * 4u, 0, 0);
        const uint32_t cnt1 = __builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)((s0 + KPT - 1) >> msh) * 4u, 0, 0);
        uint64_t v[KPT];
        if constexpr (KPT == 1) {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rc, (uint32_t)s0 * 8u, 0, 0);
            v[0] = ((uint64_t)x[1] << 32) | x[0];
        } else {
#pragma unroll
            for (int j = 0; j < KPT; j += 2) {
                const u32x4 x = ld_buf128(rc, (uint32_t)(s0 + j) * 8u);
                v[j] = ((uint64_t)x[1] << 32) | x[0];
                v[j + 1] = ((uint64_t)x[3] << 32) | x[2];
            }
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int s = s0 + j;
            const uint32_t cnt = ((s >> msh) == tile0 ? cnt0 : cnt1) & (uint32_t)(kIncomplete - 1);
            const bool ok = s < M && (uint32_t)(s & (m - 1)) < cnt;
            key[j] = ok ? (uint32_t)(v[j] >> 32) : 0u;
        }
    }
    const uint32_t picks = select_top_slots<kBNT, KPT>(key, (uint32_t)select_k, T);
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kBNT>((uint32_t)__popc(picks), T.S.scan, &total);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if ((picks >> j) & 1u) atomicAdd(&tpicked[(s0 + j) >> msh], 1u);
    lds_barrier();
    // A tile that dropped pools and had all m kept ones selected cannot vouch
    // for the pools it dropped.
    for (int c = tid; c < ntiles; c += kBNT)
        if ((cn[c] & kIncomplete) && tpicked[c] == (uint32_t)m) fail = 1;
    lds_barrier();
    if (fail) {
        topk_stream_exact<kBNT>(scores + (int64_t)t * stride, n, select_k, T.S, sel, kMaxK);
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool pk = (picks >> j) & 1u;
            if (pk && pos < (uint32_t)kMaxK) sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)cr[s0 + j]);
            pos += pk;
        }
    }
    lds_barrier();
    emit_selection<kBNT>(sel, select_k, select_k, t, b, f, qp, n_vis, e);
}

// Rows of at most 1024 KPT pools: thread i holds pools i KPT .. i KPT + KPT - 1
// as keys (0 past the row's visible pools), select_top_slots picks the best
// K, and a block scan places them in id order.  The row's scores are read
// through a descriptor bounded to the visible pools, in 16-byte loads when
// the row starts on 16 bytes (VEC), else one score at a time.
template <int KPT, bool VEC>
__global__ __launch_bounds__(kBNT) void k_topk_direct(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int stride, int select_k, Emit e) {
    static_assert(KPT % 4 == 0, "whole 16-byte loads");
    __shared__ TopSelShared<kBNT, KPT> T;
    __shared__ int32_t sel[kMaxK];
    const int t = blockIdx.x, tid = threadIdx.x;
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int n = min(n_vis, stride);
    if (n <= select_k) {                                     // every visible pool is selected
        emit_selection<kBNT>(nullptr, n, select_k, t, b, f, qp, n_vis, e);
        return;
    }
    const int s0 = tid * KPT;
    uint32_t key[KPT];
    {
        // (VEC: the range is rounded up to whole 16-byte loads, still inside
        // the row as the stride is a multiple of 4; slots past n are masked)
        const uint32_t nr = VEC ? (uint32_t)((n + 3) & ~3) : (uint32_t)n;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scores + (int64_t)t * stride, nr * 4u);
        float v[KPT];
        if constexpr (VEC) {
#pragma unroll
            for (int j = 0; j < KPT; j += 4) {
                const u32x4 x = ld_buf128(rs, (uint32_t)(s0 + j) * 4u);
#pragma unroll
                for (int u = 0; u < 4; ++u) v[j + u] = __uint_as_float(x[u]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(s0 + j) * 4u, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = s0 + j < n ? f32_key(v[j]) : 0u;
    }
    const SlotMask<KPT> picks = select_top_slots<kBNT, KPT>(key, (uint32_t)select_k, T);
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kBNT>((uint32_t)__popcll((unsigned long long)picks), T.S.scan, &total);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool pk = (picks >> j) & 1u;
        if (pk && pos < (uint32_t)kMaxK) sel[pos] = s0 + j;
        pos += pk;
    }
    lds_barrier();
    emit_selection<kBNT>(sel, select_k, select_k, t, b, f, qp, n_vis, e);
}

// Stage B over 64-pool group lists written by the scoring pass: one
// 1024-thread workgroup per row (8 list slots per thread, so a thread's slots
// lie in one group), select_from_groups, then the outputs.
__global__ __launch_bounds__(kBNT) void k_topk_groups(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int stride, int select_k,
    const uint64_t* __restrict__ cand, const int32_t* __restrict__ cand_n, Emit e) {
    static_assert(kBNT == kMaxGroups, "one group count per thread");
    __shared__ GroupSelCore<kBNT> G;
    __shared__ int32_t sel[kGroupMaxK];
    const int t = blockIdx.x;
    const GroupQuery g = select_from_groups<kBNT>(G, sel, scores, first_valid, q_seq, q_pos,
                                                  e.indices ? e.row_base : nullptr, stride, select_k, cand, cand_n, t,
                                                  [] {}, [] {});
    emit_selection<kBNT>(g.listed ? sel : nullptr, g.K, select_k, t, g.b, g.f, g.qp, g.n_vis, e, g.rb);
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_topk_groups(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                              const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                              int32_t* indices, const void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const uint64_t* cand = reinterpret_cast<const uint64_t*>(ws);
    const int32_t* cand_n = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(ws) +
                                                             ((size_t)T * dsa::kGroupCandCap * 8 + 255) / 256 * 256);
    const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
    hipLaunchKernelGGL(dsa::k_topk_groups, dim3((unsigned)T), dim3(dsa::kBNT), 0, s, scores, seqs.first_valid,
                       q_seq, q_pos, stride, d.index_topk / d.kpool, cand, cand_n, e);
    return hipGetLastError();
}


static int topk_tiles(int32_t stride) { return (int)cdiv(stride, dsa::kTile); }

static size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }

bool topk_direct(int32_t stride) { return stride <= dsa::kDirectPools; }

bool topk_supported(const dsa_dims& d, int32_t stride) {
    const int sk = d.index_topk / d.kpool;
    return sk <= dsa::kMaxK && topk_tiles(stride) <= dsa::kMaxTiles &&
           dsa::max_row_slots(sk, topk_tiles(stride)) <= (int64_t)dsa::kMaxKpt * dsa::kBNT;
}

size_t topk_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride) {
    if (T <= 0 || stride <= 0 || topk_direct(stride)) return 0;
    const int sk = d.index_topk / d.kpool;
    const int nt = topk_tiles(stride);
    return r256((size_t)T * (size_t)dsa::cand_row_cap(sk, nt) * 8) + r256((size_t)T * nt * 4);
}

hipError_t launch_topk(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                       int32_t* indices, void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int sk = d.index_topk / d.kpool;
    if (topk_direct(stride)) {
        const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
        if (stride % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0)
            hipLaunchKernelGGL((dsa::k_topk_direct<dsa::kDirectKpt, true>), dim3((unsigned)T), dim3(dsa::kBNT), 0, s,
                               scores, seqs.first_valid, q_seq, q_pos, stride, sk, e);
        else
            hipLaunchKernelGGL((dsa::k_topk_direct<dsa::kDirectKpt, false>), dim3((unsigned)T), dim3(dsa::kBNT), 0, s,
                               scores, seqs.first_valid, q_seq, q_pos, stride, sk, e);
        return hipGetLastError();
    }
    const int nt = topk_tiles(stride);
    const int64_t cap = dsa::cand_row_cap(sk, nt);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
    int32_t* cand_n = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + r256((size_t)T * cap * 8));
    const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
    hipLaunchKernelGGL(dsa::k_topk_tiles, dim3((unsigned)nt, (unsigned)T), dim3(dsa::kTile), 0, s, scores,
                       stride, seqs.first_valid, q_seq, q_pos, sk, cap, nt, cand, cand_n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int kpt = (int)cdiv(dsa::max_row_slots(sk, nt), dsa::kBNT);     // <= kMaxKpt (topk_supported)
#define DSA_ROWS(KPT)                                                                                     \
    hipLaunchKernelGGL((dsa::k_topk_rows<KPT>), dim3((unsigned)T), dim3(dsa::kBNT), 0, s, scores,          \
                       seqs.first_valid, q_seq, q_pos, stride, sk, cap, nt, cand, cand_n, e)
    if (kpt <= 1) DSA_ROWS(1);
    else if (kpt <= 2) DSA_ROWS(2);
    else if (kpt <= 4) DSA_ROWS(4);
    else if (kpt <= 8) DSA_ROWS(8);
    else if (kpt <= dsa::kMaxKpt) DSA_ROWS(16);
    else return hipErrorInvalidValue;
#undef DSA_ROWS
    return hipGetLastError();
}

}  // namespace dsa_host
