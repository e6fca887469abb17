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
// The K-th largest key is found by range bucketing in LDS: each pass
// histograms the keys inside [lo, hi] into one bucket per thread, of width
// 2^sh (the key offset shifted right), keeps the bucket that holds rank K and
// narrows [lo, hi] to it, until that bucket is taken whole or one key value is
// left, whose first `need` occurrences in id order are taken.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "topk_core.h"

namespace dsa {

constexpr int kTile = 256;                  // pools per stage-A workgroup
constexpr int kBNT = 1024;
constexpr int kMaxK = 1024;                 // select_k limit
constexpr int kMaxTiles = 1024;             // 262,144 pools per row
constexpr int kMaxCand = 32 * kBNT;         // stage-B capacity
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
// when ntiles < 5 K / 256).
__host__ __device__ inline int64_t cand_row_cap(int select_k, int ntiles_max) {
    return 16LL * ntiles_max + 5LL * select_k + 256;
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

// Exact selection straight from the row's scores (used when the tile lists
// cannot prove they hold the answer): MSB-first radix select, 8 bits a pass,
// then one ordered pass that takes every key above the K-th and the first
// `need` keys equal to it.  Writes K ids, ascending, to sel.
template <int NT>
__device__ __noinline__ void topk_stream_exact(const float* __restrict__ row, int n, int K, SelShared<NT>& S, int32_t* sel) {
    static_assert(NT >= 256, "one thread per digit");
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K, total;
    for (int d = 3; d >= 0; --d) {
        if (tid < 256) S.hist[0][tid] = 0u;
        lds_barrier();
        for (int i = tid; i < n; i += NT) {
            const uint32_t k = f32_key(row[i]);
            if ((k & mask) == prefix) atomicAdd(&S.hist[0][(k >> (8 * d)) & 0xFFu], 1u);
        }
        lds_barrier();
        const uint32_t h = tid < 256 ? S.hist[0][255 - tid] : 0u;    // descending digits
        const uint32_t above = block_exclusive_scan<NT>(h, S.scan, &total);
        if (tid < 256 && above < need && need <= above + h) {
            S.bin[0] = 255u - (uint32_t)tid;
            S.above[0] = above;
        }
        lds_barrier();
        need -= S.above[0];
        prefix |= S.bin[0] << (8 * d);
        mask |= 0xFFu << (8 * d);
        lds_barrier();
    }
    uint32_t out_base = 0u, eq_base = 0u;
    for (int i0 = 0; i0 < n; i0 += NT) {
        const int i = i0 + tid;
        const uint32_t k = i < n ? f32_key(row[i]) : 0u;
        const uint32_t gt = (i < n && k > prefix) ? 1u : 0u;
        const uint32_t eq = (i < n && k == prefix) ? 1u : 0u;
        uint32_t eq_tot, pick_tot;
        const uint32_t eq_rank = eq_base + block_exclusive_scan<NT>(eq, S.scan, &eq_tot);
        const uint32_t pick = gt | ((eq && eq_rank < need) ? 1u : 0u);
        const uint32_t pos = out_base + block_exclusive_scan<NT>(pick, S.scan, &pick_tot);
        if (pick && pos < (uint32_t)kMaxK) sel[pos] = i;
        out_base += pick_tot;
        eq_base += eq_tot;
    }
}

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
    uint32_t key[KPT];
    int32_t id[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int s = s0 + j;
        key[j] = 0u;
        id[j] = 0;
        if (s < M && (s & (m - 1)) < (cn[s >> msh] & (kIncomplete - 1))) {
            const uint64_t v = cr[s];
            key[j] = (uint32_t)(v >> 32);
            id[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
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
        topk_stream_exact<kBNT>(scores + (int64_t)t * stride, n, select_k, T.S, sel);
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool pk = (picks >> j) & 1u;
            if (pk && pos < (uint32_t)kMaxK) sel[pos] = id[j];
            pos += pk;
        }
    }
    lds_barrier();
    emit_selection<kBNT>(sel, select_k, select_k, t, b, f, qp, n_vis, e);
}

// Stage B over 64-pool group lists written by the scoring pass (one
// 1024-thread workgroup per row; 8 list slots per thread, so a thread's slots
// lie in one group).  The selection is the one select_top_slots makes (range
// bucketing, then an exact rank of the boundary bucket), arranged around as
// few workgroup barriers as the data flow allows, since at one workgroup per
// row the barriers are the cost:
//   A  list slots are valid by position alone (empty slots hold key 0), so
//      the per-wave min/max is published with the group counts;
//   B, C per bucketing pass: the histogram, then wave 0's search of it;
//   D  the boundary bucket's entries: each thread then ranks its own;
//   E  per-wave pick counts (output order) and the list check, both local:
//      a group that dropped pools and has all m kept entries picked fails
//      it (the exact pass over the scores then decides);
//   F  the selection in LDS, then the index list.
struct GroupSel {
    uint32_t hist[kSelPasses][kBNT];
    uint32_t mm[2 * kBNT / 64];
    uint32_t res[4];
    uint32_t nb, fail;
    uint64_t bent[kBoundCap];                // boundary entries: key << 32 | ~slot, 0 past the end
    uint32_t wsum[kBNT / 64];
    uint32_t gcount[kMaxGroups];
    int32_t sel[kGroupMaxK];
    SelShared<kBNT> S;                       // the exact pass
};

__global__ __launch_bounds__(kBNT) void k_topk_groups(
    const float* __restrict__ scores, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int stride, int select_k,
    const uint64_t* __restrict__ cand, const int32_t* __restrict__ cand_n, Emit e) {
    constexpr int KPT = kGroupCandCap / kBNT, NW = kBNT / 64, NB = kBNT, PER = NB / 64;
    constexpr int BITS = log2_of<NB>();
    __shared__ GroupSel G;
    static_assert(KPT == 8 && kBNT == kMaxGroups, "8 list slots and one group count per thread");
    static_assert(PER == 16 && kBoundCap % 8 == 0, "one 16-lane row per bucket run; rank in steps of 8");
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int s0 = tid * KPT;
    // every load at once, before the row geometry they do not depend on: this
    // thread's group count and its KPT slots
    const uint32_t gc = (uint32_t)cand_n[(int64_t)t * kMaxGroups + tid];
    uint64_t raw[KPT];
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(cand + (int64_t)t * kGroupCandCap + s0);
#pragma unroll
        for (int j = 0; j < KPT; j += 2) {
            const u32x4 v = src[j / 2];
            raw[j] = ((uint64_t)v[1] << 32) | v[0];
            raw[j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    }
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int64_t rb = e.indices ? e.row_base[b] : 0;
    const int n = min(n_vis, stride);
    if (n <= select_k) {
        emit_selection<kBNT>(nullptr, n, select_k, t, b, f, qp, n_vis, e, rb);
        return;
    }
    const int groups = (n + kGroupPools - 1) / kGroupPools;
    const int m = group_quota(select_k, n);
    const int msh = __ffs(m) - 1;
    const int M = groups * m;
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = s0 + j < M ? (uint32_t)(raw[j] >> 32) : 0u;

    // ---- A: counts, cleared histograms, per-wave min (present keys) / max
    G.gcount[tid] = gc;
#pragma unroll
    for (int i = 0; i < kSelPasses; ++i) G.hist[i][tid] = 0u;
    if (tid == 0) {
        G.nb = 0u;
        G.fail = 0u;
    }
    if (tid < kBoundCap) G.bent[tid] = 0ull;
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (key[j]) lo = min(lo, key[j]);
        hi = max(hi, key[j]);
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        G.mm[2 * w] = lo;
        G.mm[2 * w + 1] = hi;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        lo = min(lo, G.mm[2 * i]);
        hi = max(hi, G.mm[2 * i + 1]);
    }

    // ---- B, C: bucketing passes
    const uint32_t target = (uint32_t)select_k;
    uint32_t krem = target, cnt = 0xFFFFFFFFu;
    bool whole = false;
#pragma unroll 1
    for (int pass = 0; pass < kSelPasses && lo < hi && cnt > (uint32_t)kBoundCap; ++pass) {
        uint32_t* H = G.hist[pass];
        const int sh = bit_len<uint32_t>((hi - lo) >> BITS);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t k = key[j];
            if (k >= lo && k <= hi) atomicAdd(&H[(k - lo) >> sh], 1u);
        }
        lds_barrier();
        if (w == 0) {
            // bucket d (descending: bucket NB-1-d) holding rank krem; lane l
            // sums d in [l PER, (l+1) PER), read in a rotated, conflict-free order
            uint32_t lsum = 0u;
#pragma unroll
            for (int i = 0; i < PER; ++i) lsum += H[NB - 1 - (lane * PER + ((i + lane / (64 / PER)) & (PER - 1)))];
            const uint32_t incl = wave_incl_sum_u32(lsum), excl = incl - lsum;
            const unsigned long long hit = __ballot(excl < krem && krem <= incl);
            uint32_t d = 0u, above = 0u, c = 0u, none = 1u;
            if (hit != 0ull) {
                // within lane L's run: lane i of each row reads its bucket L PER + i,
                // a row scan gives the running counts, the first that reaches krem wins
                none = 0u;
                const int L = __ffsll((long long)hit) - 1;
                const uint32_t acc = __builtin_amdgcn_readlane(excl, L);
                const uint32_t v = H[NB - 1 - (L * PER + (lane & (PER - 1)))];
                const uint32_t run = row_incl_sum_u32(v);
                const int i = __ffsll((long long)(__ballot(krem <= acc + run) & 0xFFFFull)) - 1;
                d = (uint32_t)(L * PER + i);
                c = __builtin_amdgcn_readlane(v, i);
                above = acc + __builtin_amdgcn_readlane(run, i) - c;
            }
            if (lane == 0) {
                G.res[0] = d;
                G.res[1] = above;
                G.res[2] = c;
                G.res[3] = none;
            }
        }
        lds_barrier();
        if (G.res[3]) {                      // fewer present keys than the target: all of them
            whole = true;
            break;
        }
        krem -= G.res[1];
        cnt = G.res[2];
        const uint32_t nlo = lo + ((NB - 1 - G.res[0]) << sh);
        const uint32_t nhi = nlo + ((1u << sh) - 1u);
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
        if (cnt == krem) {
            whole = true;
            break;
        }
    }
    if (lo == hi && cnt == 0xFFFFFFFFu) {    // every present key equal (or one key)
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] == lo ? 1u : 0u;
        uint32_t tot;
        block_exclusive_scan<kBNT>(c, G.S.scan, &tot);
        cnt = tot;
        whole = tot == krem;
    }
    uint32_t picks = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (key[j] > hi || (whole && key[j] != 0u && key[j] >= lo && key[j] <= hi)) picks |= 1u << j;

    // ---- D: the boundary bucket [lo, hi]; each thread ranks its own entries
    if (!whole) {
        if (cnt <= (uint32_t)kBoundCap) {
            // entry = key << 32 | ~slot: a larger entry is a larger key, or an
            // equal key at a lower slot, so an entry's rank is the number of
            // larger entries; one atomic per wave places this wave's entries
            uint32_t mine = 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) mine += (key[j] != 0u && key[j] >= lo && key[j] <= hi) ? 1u : 0u;
            const uint32_t wrun = wave_incl_sum_u32(mine);
            uint32_t wbase = 0u;
            if (lane == 63 && wrun != 0u) wbase = atomicAdd(&G.nb, wrun);
            const uint32_t e0 = __builtin_amdgcn_readlane(wbase, 63) + wrun - mine;
            if (mine) {
                uint32_t e = e0;
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    if (key[j] != 0u && key[j] >= lo && key[j] <= hi) {
                        G.bent[e] = ((uint64_t)key[j] << 32) | (0xFFFFFFFFu - (uint32_t)(s0 + j));
                        ++e;
                    }
                }
            }
            lds_barrier();
            // this thread's entries are [e0, e0 + mine); entries past nb are 0
            const uint32_t nb8 = (G.nb + 7u) & ~7u;
            for (uint32_t me = e0; me < e0 + mine; ++me) {
                const uint64_t mk = G.bent[me];
                uint32_t rank = 0;
                for (uint32_t i = 0; i < nb8; i += 8) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) rank += G.bent[i + u] > mk ? 1u : 0u;
                }
                if (rank < krem) picks |= 1u << ((0xFFFFFFFFu - (uint32_t)mk) - (uint32_t)s0);
            }
        } else {
            // more than kBoundCap equal keys (lo == hi): the first krem in slot order
            uint32_t c = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) c += (key[j] != 0u && key[j] == lo) ? 1u : 0u;
            uint32_t tot;
            const uint32_t before = block_exclusive_scan<kBNT>(c, G.S.scan, &tot);
            uint32_t take = krem > before ? min(krem - before, c) : 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                if (key[j] != 0u && key[j] == lo && take > 0u) {
                    picks |= 1u << j;
                    --take;
                }
            }
        }
    }

    // ---- E: output positions (per-wave counts) and the list check
    const uint32_t c = (uint32_t)__popc(picks);
    const uint32_t incl = wave_incl_sum_u32(c);
    if (lane == 63) G.wsum[w] = incl;
    {
        // threads tpg * g' .. tpg * g' + tpg - 1 of this wave hold group g's m slots
        const int tpg = m >> 3;
        const unsigned long long full = __ballot(picks == 0xFFu);
        const int l0 = lane & ~(tpg - 1);
        const unsigned long long gm = ((tpg >= 64 ? ~0ull : ((1ull << tpg) - 1ull))) << l0;
        const bool bad = (lane & (tpg - 1)) == 0 && s0 < M && (G.gcount[s0 >> msh] & kGroupDropped) &&
                         (full & gm) == gm;
        if (__ballot(bad) != 0ull && lane == 0) G.fail = 1u;
    }
    lds_barrier();
    uint32_t pos = incl - c;
#pragma unroll
    for (int i = 0; i < NW; ++i) pos += i < w ? G.wsum[i] : 0u;
    if (G.fail) {
        topk_stream_exact<kBNT>(scores + (int64_t)t * stride, n, select_k, G.S, G.sel);
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if ((picks >> j) & 1u) {
                if (pos < (uint32_t)kGroupMaxK) G.sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)raw[j]);
                ++pos;
            }
        }
    }
    // ---- F
    lds_barrier();
    emit_selection<kBNT>(G.sel, select_k, select_k, t, b, f, qp, n_vis, e, rb);
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

bool topk_supported(const dsa_dims& d, int32_t stride) {
    const int sk = d.index_topk / d.kpool;
    return sk <= dsa::kMaxK && topk_tiles(stride) <= dsa::kMaxTiles &&
           dsa::cand_row_cap(sk, topk_tiles(stride)) <= dsa::kMaxCand;
}

size_t topk_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride) {
    if (T <= 0 || stride <= 0) return 0;
    const int sk = d.index_topk / d.kpool;
    const int nt = topk_tiles(stride);
    return r256((size_t)T * (size_t)dsa::cand_row_cap(sk, nt) * 8) + r256((size_t)T * nt * 4);
}

hipError_t launch_topk(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                       int32_t* indices, void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int sk = d.index_topk / d.kpool;
    const int nt = topk_tiles(stride);
    const int64_t cap = dsa::cand_row_cap(sk, nt);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
    int32_t* cand_n = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + r256((size_t)T * cap * 8));
    const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
    hipLaunchKernelGGL(dsa::k_topk_tiles, dim3((unsigned)nt, (unsigned)T), dim3(dsa::kTile), 0, s, scores,
                       stride, seqs.first_valid, q_seq, q_pos, sk, cap, nt, cand, cand_n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // Slots per row are at most ntiles * tile_quota(ntiles) <= cap.
    const int kpt = (int)cdiv(cap, dsa::kBNT);
#define DSA_ROWS(KPT)                                                                                     \
    hipLaunchKernelGGL((dsa::k_topk_rows<KPT>), dim3((unsigned)T), dim3(dsa::kBNT), 0, s, scores,          \
                       seqs.first_valid, q_seq, q_pos, stride, sk, cap, nt, cand, cand_n, e)
    if (kpt <= 1) DSA_ROWS(1);
    else if (kpt <= 2) DSA_ROWS(2);
    else if (kpt <= 4) DSA_ROWS(4);
    else if (kpt <= 8) DSA_ROWS(8);
    else if (kpt <= 16) DSA_ROWS(16);
    else DSA_ROWS(32);
#undef DSA_ROWS
    return hipGetLastError();
}

}  // namespace dsa_host
