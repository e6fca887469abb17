// The best K pools of a row from the group lists (64 pools a group, 256 in
// rows past 65,536 pools) the scoring pass keeps ([Ref] Functions: topk_pools; [Flash] Stream C: indexer_topk512),
// as a workgroup-wide device function: k_topk_groups runs it on 1024
// threads, the selection + attention launch on the 512 threads of its
// attention workgroups.  Both make the same selection: the K best by
// (score desc, pool id asc), ascending ids.
//
// The steps are arranged around as few workgroup barriers as the data flow
// allows, since at one workgroup per row the barriers are the cost:
//   A  list slots are valid by position alone (empty slots hold key 0), so
//      the per-wave min/max is published with the group counts;
//   B, C per bucketing pass: the histogram, then the search of it (by every
//      wave when there are at most 8, so C needs no barrier of its own);
//   D  the boundary bucket's entries: each thread then ranks its own;
//   E  per-wave pick counts (output order) and the list check, both local:
//      a group that dropped pools and has all m kept entries picked fails
//      it (an exact pass over the row's scores then decides);
//   F  the selection in LDS.
#pragma once
#include "dsa_common.h"
#include "topk_core.h"

namespace dsa {

constexpr int kSelBuckets = 1024;          // buckets per bucketing pass

// Exact selection straight from the row's scores (used when the candidate
// lists cannot prove they hold the answer): MSB-first radix select, 8 bits a
// pass, then one ordered pass that takes every key above the K-th and the
// first `need` keys equal to it.  Writes K ids, ascending, to sel (of cap
// entries).
template <int NT>
__device__ __noinline__ void topk_stream_exact(const float* __restrict__ row, int n, int K, SelShared<NT>& S,
                                               int32_t* sel, int cap) {
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
        if (pick && pos < (uint32_t)cap) sel[pos] = i;
        out_base += pick_tot;
        eq_base += eq_tot;
    }
}

// Workgroup state of the selection; the selected ids live outside it, so a
// caller may reuse this memory once the selection has returned.
template <int NT>
struct GroupSelCore {
    uint32_t hist[kSelPasses][kSelBuckets + 64];   // + one spill bucket per lane
    uint32_t mm[2 * NT / 64];
    uint32_t res[4];
    uint32_t nb, fail;
    uint64_t bent[kBoundCap];                // boundary entries: key << 32 | ~slot, 0 past the end
    uint32_t wsum[NT / 64];
    uint32_t gcount[kMaxGroups];
    SelShared<NT> S;                         // the exact pass
};

// The query's geometry and its selection: K ids, in sel when `listed`,
// otherwise (every visible pool selected) simply 0 .. K-1.
struct GroupQuery {
    int b, f, qp, n_vis;
    int64_t rb;                              // row_base[b] (0 without row_base)
    int K;
    bool listed;
};

// Row t's selection from its group lists cand / cand_n.  Every thread of the
// workgroup must call it.  When `listed`, it returns after a workgroup
// barrier with sel[0 .. K) written and G no longer in use; otherwise it
// returns before touching G or sel (and without a barrier).  issued() runs
// right after the group lists' loads are issued (the caller's own early
// loads go there, behind them); staged() runs just before the last barrier
// (LDS writes of the caller's outside G ride on it).
template <int NT, class Issued, class Staged>
__device__ __forceinline__ GroupQuery select_from_groups(
    GroupSelCore<NT>& G, int32_t* sel, const float* __restrict__ scores, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, const int64_t* __restrict__ row_base,
    int stride, int select_k, const uint64_t* __restrict__ cand, const int32_t* __restrict__ cand_n, int t,
    Issued issued, Staged staged) {
    constexpr int KPT = kGroupCandCap / NT, NW = NT / 64, NB = kSelBuckets, PER = NB / 64;
    constexpr int GPT = kMaxGroups / NT;     // group counts per thread
    constexpr int BITS = log2_of<NB>();
    constexpr uint32_t ALL = (1u << KPT) - 1u;
    constexpr bool kWaveSearch = NW <= 8;
    static_assert(KPT >= 8 && KPT <= 16 && GPT * NT == kMaxGroups, "8 or 16 list slots per thread");
    static_assert(PER == 16 && kBoundCap % 8 == 0, "one 16-lane row per bucket run; rank in steps of 8");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int s0 = tid * KPT;
    // every load at once, before the row geometry they do not depend on: this
    // thread's group counts and its KPT slots
    uint32_t gc[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) gc[i] = (uint32_t)cand_n[(int64_t)t * kMaxGroups + tid + NT * i];
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
    __builtin_amdgcn_sched_barrier(0);       // the list loads leave first
    issued();
    GroupQuery g;
    query_geom(first_valid, q_seq, q_pos, t, g.b, g.f, g.qp, g.n_vis);
    g.rb = row_base ? row_base[g.b] : 0;
    const int n = min(g.n_vis, stride);
    if (n <= select_k) {
        g.K = n;
        g.listed = false;
        return g;
    }
    g.K = select_k;
    g.listed = true;
    const int gp = group_pools(n);
    const int groups = (n + gp - 1) / gp;
    const int m = group_quota(select_k, n);
    const int msh = __ffs(m) - 1;
    const int M = groups * m;
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = s0 + j < M ? (uint32_t)(raw[j] >> 32) : 0u;

    // ---- A: counts, cleared histograms, per-wave min (present keys) / max
#pragma unroll
    for (int i = 0; i < GPT; ++i) G.gcount[tid + NT * i] = gc[i];
#pragma unroll
    for (int p = 0; p < kSelPasses; ++p)
#pragma unroll
        for (int i = 0; i < NB / NT; ++i) G.hist[p][tid + NT * i] = 0u;
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
        const uint32_t span = hi - lo;
        const int sh = bit_len<uint32_t>(span >> BITS);
        // (key - lo) <= span is lo <= key <= hi (key 0 wraps above span, as
        // lo >= 1); a key outside goes to this lane's spill bucket, so the
        // loop needs no branch
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t off = key[j] - lo;
            atomicAdd(&H[off <= span ? (off >> sh) : (uint32_t)(NB + lane)], 1u);
        }
        lds_barrier();
        // bucket d (descending: bucket NB-1-d) holding rank krem; lane l sums
        // d in [l PER, (l+1) PER), read in a rotated, conflict-free order.
        // With at most 8 waves every wave searches (the same answer, no second
        // barrier); with more, wave 0 searches and publishes the result.
        uint32_t r_d = 0u, r_above = 0u, r_c = 0u, r_none = 1u;
        if (kWaveSearch || w == 0) {
            uint32_t lsum = 0u;
#pragma unroll
            for (int i = 0; i < PER; ++i) lsum += H[NB - 1 - (lane * PER + ((i + lane / (64 / PER)) & (PER - 1)))];
            const uint32_t incl = wave_incl_sum_u32(lsum), excl = incl - lsum;
            const unsigned long long hit = __ballot(excl < krem && krem <= incl);
            if (hit != 0ull) {
                // within lane L's run: lane i of each row reads its bucket L PER + i,
                // a row scan gives the running counts, the first that reaches krem wins
                r_none = 0u;
                const int L = __ffsll((long long)hit) - 1;
                const uint32_t acc = __builtin_amdgcn_readlane(excl, L);
                const uint32_t v = H[NB - 1 - (L * PER + (lane & (PER - 1)))];
                const uint32_t run = row_incl_sum_u32(v);
                const int i = __ffsll((long long)(__ballot(krem <= acc + run) & 0xFFFFull)) - 1;
                r_d = (uint32_t)(L * PER + i);
                r_c = __builtin_amdgcn_readlane(v, i);
                r_above = acc + __builtin_amdgcn_readlane(run, i) - r_c;
            }
            if (!kWaveSearch && lane == 0) {
                G.res[0] = r_d;
                G.res[1] = r_above;
                G.res[2] = r_c;
                G.res[3] = r_none;
            }
        }
        if constexpr (!kWaveSearch) {
            lds_barrier();
            r_d = G.res[0];
            r_above = G.res[1];
            r_c = G.res[2];
            r_none = G.res[3];
        }
        if (r_none) {                        // fewer present keys than the target: all of them
            whole = true;
            break;
        }
        krem -= r_above;
        cnt = r_c;
        const uint32_t nlo = lo + ((NB - 1 - r_d) << sh);
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
        block_exclusive_scan<NT>(c, G.S.scan, &tot);
        cnt = tot;
        whole = tot == krem;
    }
    // every key above hi, and the whole of [lo, hi] when `whole` (lo >= 1
    // whenever a key is present, so absent keys are never picked)
    uint32_t picks = 0u;
    if (whole) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) picks |= (key[j] >= lo ? 1u : 0u) << j;
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) picks |= (key[j] > hi ? 1u : 0u) << j;
    }

    // ---- D: the boundary bucket [lo, hi]; each thread ranks its own entries
    if (!whole) {
        if (cnt <= (uint32_t)kBoundCap) {
            // entry = key << 32 | ~slot: a larger entry is a larger key, or an
            // equal key at a lower slot, so an entry's rank is the number of
            // larger entries; one atomic per wave places this wave's entries
            const uint32_t span = hi - lo;
            uint32_t mine = 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) mine += key[j] - lo <= span ? 1u : 0u;
            const uint32_t wrun = wave_incl_sum_u32(mine);
            uint32_t wbase = 0u;
            if (lane == 63 && wrun != 0u) wbase = atomicAdd(&G.nb, wrun);
            const uint32_t e0 = __builtin_amdgcn_readlane(wbase, 63) + wrun - mine;
            if (mine) {
                uint32_t e = e0;
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    if (key[j] - lo <= span) {
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
            const uint32_t before = block_exclusive_scan<NT>(c, G.S.scan, &tot);
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
        bool bad = false;
        if (m >= KPT) {
            // threads tpg * g' .. tpg * g' + tpg - 1 of this wave hold group g's m slots
            const int tpg = m / KPT;
            const unsigned long long full = __ballot(picks == ALL);
            const int l0 = lane & ~(tpg - 1);
            const unsigned long long gm = ((tpg >= 64 ? ~0ull : ((1ull << tpg) - 1ull))) << l0;
            bad = (lane & (tpg - 1)) == 0 && s0 < M && (G.gcount[s0 >> msh] & kGroupDropped) && (full & gm) == gm;
        } else {
            // KPT / m whole groups per thread
            const uint32_t gmask = (1u << m) - 1u;
            for (int i = 0; i < KPT; i += m)
                bad = bad || (s0 + i < M && (G.gcount[(s0 + i) >> msh] & kGroupDropped) &&
                              ((picks >> i) & gmask) == gmask);
        }
        if (__ballot(bad) != 0ull && lane == 0) G.fail = 1u;
    }
    lds_barrier();
    uint32_t pos = incl - c;
#pragma unroll
    for (int i = 0; i < NW; ++i) pos += i < w ? G.wsum[i] : 0u;
    if (G.fail) {
        topk_stream_exact<NT>(scores + (int64_t)t * stride, n, select_k, G.S, sel, kGroupMaxK);
    } else {
        // slot j's output position is pos + (picks below j); a slot not
        // picked writes its lane's spill word of a histogram, so the stores
        // need no branch
        uint32_t* spill = &G.hist[0][NB + lane];
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t pj = pos + (uint32_t)__popc(picks & ((1u << j) - 1u));
            const bool wr = ((picks >> j) & 1u) && pj < (uint32_t)kGroupMaxK;
            *(wr ? reinterpret_cast<uint32_t*>(&sel[pj]) : spill) = 0xFFFFFFFFu - (uint32_t)raw[j];
        }
    }
    // ---- F
    staged();
    lds_barrier();
    return g;
}

}  // namespace dsa
