// Selection machinery shared by the top-k kernels and the fused decode step:
// query geometry, order-preserving keys, block min/max, range-bucket select
// and order-preserving compaction.  The design notes are at the top of
// topk.hip.
#pragma once
#include <type_traits>

#include "dsa_common.h"

namespace dsa {

struct Emit {
    int32_t* pool_ids;        // [T, select_k] or null
    int32_t* indices;         // [T, W] or null
    const int64_t* row_base;
    int W;
};

__device__ __forceinline__ void query_geom(const int32_t* first_valid, const int32_t* q_seq,
                                           const int32_t* q_pos, int t, int& b, int& f, int& qp,
                                           int& n_vis) {
    b = q_seq[t];
    f = first_valid[b];
    qp = q_pos[t];
    n_vis = qp >= f ? (qp - f + 1) >> 2 : 0;
}

// Write K ascending ids (sel[0..K), or 0..K-1 when sel is null) as pool ids
// (-1 padded) and/or as the expanded index list.  No barrier inside.
// rb: row_base[b] when the caller loaded it already (-1: load it here).
template <int NT>
__device__ __forceinline__ void emit_selection(const int32_t* sel, int K, int select_k, int t, int b,
                                               int f, int qp, int n_vis, const Emit& e, int64_t rb_pre = -1) {
    const int tid = threadIdx.x;
    if (e.pool_ids) {
        int32_t* out = e.pool_ids + (int64_t)t * select_k;
        for (int i = tid; i < select_k; i += NT) out[i] = i < K ? (sel ? sel[i] : i) : -1;
    }
    if (e.indices) {
        const int64_t rb = rb_pre >= 0 ? rb_pre : e.row_base[b];
        const int nsel = 4 * K;
        const int tail = qp >= f ? (qp - f + 1) - 4 * n_vis : 0;
        int32_t* out = e.indices + (int64_t)t * e.W;
        for (int j = tid; j < e.W; j += NT) {
            int64_t v = -1;
            if (j < nsel) v = rb + f + 4 * (int64_t)(sel ? sel[j >> 2] : (j >> 2)) + (j & 3);
            else if (j < nsel + tail) v = rb + f + 4 * (int64_t)n_vis + (j - nsel);
            out[j] = (int32_t)v;
        }
    }
}

template <typename KT>
__device__ __forceinline__ KT shfl_xor_k(KT v, int o) {
    if constexpr (sizeof(KT) == 8) {
        const uint32_t lo = __shfl_xor((int)(uint32_t)v, o, 64);
        const uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), o, 64);
        return ((uint64_t)hi << 32) | lo;
    } else {
        return (KT)__shfl_xor((int)v, o, 64);
    }
}

template <typename KT>
__device__ __forceinline__ int bit_len(KT v) {
    if constexpr (sizeof(KT) == 8) return v ? 64 - __clzll((long long)v) : 0;
    else return v ? 32 - __clz((int)v) : 0;
}

// Block min (over non-zero keys) and max of register keys.
template <int NT, int KPT, typename KT>
__device__ __forceinline__ void block_min_max(const KT (&key)[KPT], KT* sh, KT& kmin, KT& kmax) {
    KT mn = ~(KT)0, mx = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (key[j]) mn = key[j] < mn ? key[j] : mn;
        mx = key[j] > mx ? key[j] : mx;
    }
    if constexpr (sizeof(KT) == 4) {
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
    } else {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const KT a = shfl_xor_k(mn, o), c = shfl_xor_k(mx, o);
            mn = a < mn ? a : mn;
            mx = c > mx ? c : mx;
        }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sh[2 * w] = mn; sh[2 * w + 1] = mx; }
    lds_barrier();
    kmin = sh[0];
    kmax = sh[1];
    for (int i = 1; i < NT / 64; ++i) {
        kmin = sh[2 * i] < kmin ? sh[2 * i] : kmin;
        kmax = sh[2 * i + 1] > kmax ? sh[2 * i + 1] : kmax;
    }
    lds_barrier();
}

// One bucket per thread: NT buckets per pass, double-buffered so the next
// pass's buckets are cleared while this pass's are read.
template <int NT>
struct SelShared {
    uint32_t hist[2][NT];
    uint32_t scan[NT / 64 + 1];
    uint32_t bin[2], above[2], cnt[2];
};

template <int N>
constexpr int log2_of() { return N == 256 ? 8 : (N == 512 ? 9 : (N == 1024 ? 10 : 11)); }

// Find the range [lo, hi] holding the rank-`target` key (absent keys are 0).
// On return every key > hi is in the top `target`; `krem` of the keys inside
// [lo, hi] complete it: all of them when `whole`, else (lo == hi) the first
// krem in id order.  Each pass cuts the span by log2(NT) bits.
template <int NT, int KPT, typename KT>
__device__ __forceinline__ void bucket_select(const KT (&key)[KPT], uint32_t target, SelShared<NT>& S,
                                              KT* mm_sh, KT& lo, KT& hi, uint32_t& krem, bool& whole) {
    constexpr int BITS = log2_of<NT>();
    const int tid = threadIdx.x;
    S.hist[0][tid] = 0u;
    S.hist[1][tid] = 0u;
    block_min_max<NT, KPT, KT>(key, mm_sh, lo, hi);          // contains the barrier that publishes the clears
    krem = target;
    whole = false;
    // The cap only bounds the loop (a 64-bit span closes in at most 8 passes).
    for (int pass = 0; pass < 8 && lo < hi; ++pass) {
        const int buf = pass & 1;
        const int sh = bit_len<KT>((hi - lo) >> BITS);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const KT k = key[j];
            if (k >= lo && k <= hi) atomicAdd(&S.hist[buf][(uint32_t)((k - lo) >> sh)], 1u);
        }
        lds_barrier();
        const uint32_t h = S.hist[buf][NT - 1 - tid];         // thread order = descending buckets
        S.hist[buf ^ 1][tid] = 0u;                            // read two passes ago; free now
        uint32_t total;
        const uint32_t above = block_exclusive_scan<NT>(h, S.scan, &total);
        if (above < krem && krem <= above + h) {
            S.bin[buf] = NT - 1 - tid;
            S.above[buf] = above;
            S.cnt[buf] = h;
        }
        lds_barrier();
        krem -= S.above[buf];
        const KT nlo = lo + ((KT)S.bin[buf] << sh);
        const KT nhi = nlo + (((KT)1 << sh) - 1);
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
        whole = S.cnt[buf] == krem;
        if (whole) break;
    }
    if (!(lo == hi && !whole)) whole = true;
}

// This thread's output slot (exclusive scan of its selected-key count) and its
// budget `take` of keys inside [lo, hi].
template <int NT, int KPT, typename KT>
__device__ __forceinline__ uint32_t compaction_slot(const KT (&key)[KPT], KT lo, KT hi, uint32_t krem,
                                                    bool whole, SelShared<NT>& S, uint32_t& take) {
    uint32_t gt = 0, in = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += key[j] > hi;
        in += key[j] >= lo && key[j] <= hi;
    }
    uint32_t total;
    take = in;
    if (!whole) {
        const uint32_t base = block_exclusive_scan<NT>(in, S.scan, &total);
        take = krem > base ? min(krem - base, in) : 0u;
    }
    return block_exclusive_scan<NT>(gt + take, S.scan, &total);
}

// ---------------------------------------------------------------- pool group candidates
// A scoring pass can keep, for each group of consecutive pools, its best m
// pools by (score desc, id asc); the union of the group lists holds the top-K
// unless a group that dropped pools has all m kept ones selected, which the
// selection checks (falling back to an exact select over the scores).  A
// group is 64 pools (one wave) in rows of at most 65,536 pools, 256 pools
// (one scoring workgroup's tile) in longer rows, so that a row never has
// more than kMaxGroups groups.
constexpr int kGroupPools = 64;
constexpr int kLongGroupPools = 256;
constexpr int kMaxGroups = 1024;
constexpr int kShortListPools = kMaxGroups * kGroupPools;       // 65,536
constexpr int kListMaxPools = kMaxGroups * kLongGroupPools;     // 262,144
constexpr int kGroupCandCap = 8192;       // kept entries per row
constexpr int kGroupMaxK = 512;
constexpr int kGroupDropped = 1 << 30;    // group count flag: the group dropped pools

__host__ __device__ __forceinline__ int group_pools(int n) { return n > kShortListPools ? kLongGroupPools : kGroupPools; }

// Kept entries per group for a row of n visible pools (n > K): a power of two
// >= lambda + 5 sqrt(lambda) + 4, lambda = G K / n being a group's mean share
// of the K (G pools a group; a group needing more than m is a > 5-sigma
// event); at least 8, at most 64 and at most kGroupCandCap / groups.
// SHORT: the caller's rows are known to be at most 65,536 pools.
template <bool SHORT = false>
__device__ __forceinline__ int group_quota(int K, int n) {
    const int gp = SHORT ? kGroupPools : group_pools(n);
    const int groups = (n + gp - 1) / gp;
    const float lam = (float)gp * (float)K / (float)n;
    const float want = lam + 5.0f * sqrtf(lam) + 4.0f;
    int m = 8;
    while ((float)m < want && m < kGroupPools) m <<= 1;
    while (m > 8 && groups * m > kGroupCandCap) m >>= 1;
    return m;
}

// The best m of a wave's `valid` keys, lane order being id order: writes
// them (key << 32 | ~id) in id order to cand[group * m ..], zeros in the
// list's remaining slots (key 0 marks an empty slot), and the count
// (| kGroupDropped when the group held more than m pools, nvalid being how
// many it held) to cand_n[group].  The best m are taken by repeated wave
// maxima for m = 8, else through the m-th largest key (32
// ballot-and-popcount steps); either way ties go to the lowest ids.  Store is
// the memory policy for the two writes.
template <class Store64, class Store32>
__device__ __forceinline__ void keep_best_keys(uint32_t key, bool valid, uint32_t id, int nvalid, int group, int m,
                                               uint64_t* cand, int32_t* cand_n, Store64 st64, Store32 st32) {
    const int lane = threadIdx.x & 63;
    const int nkeys = __popcll(__ballot(valid));
    bool pick = valid;
    if (nkeys > m && m <= 8) {
        // m = 8: take the largest remaining key 8 times (a DPP wave max, then
        // the lowest lane holding it, which drops out) -- a dozen mostly
        // vector instructions a round, where the 32-step threshold search
        // below is a chain of scalar ones that the waves of a CU would all
        // issue at once.  From m = 16 on the search is the cheaper one
        // (measured per wave: 16 rounds 2.7 us, the search 1.6 us).
        uint32_t cur = key;                     // 0: invalid or taken
        unsigned long long taken = 0ull;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t mx = wave_max_u32(cur);
            const int first = __ffsll((long long)__ballot(cur == mx)) - 1;
            taken |= 1ull << first;
            cur = lane == first ? 0u : cur;
        }
        pick = (taken >> lane) & 1ull;
    } else if (nkeys > m) {
        // x = the m-th largest key: the largest x with at least m keys >= x
        uint32_t x = 0u;
#pragma unroll
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t y = x | (1u << bit);
            if (__popcll(__ballot(key >= y)) >= m) x = y;
        }
        const unsigned long long eqm = __ballot(key == x);
        const int above = __popcll(__ballot(key > x));
        const int eq_before = popc_below(eqm);
        pick = key > x || (key == x && eq_before < m - above);
    }
    const unsigned long long pm = __ballot(pick);
    const int slot = popc_below(pm);
    const int npk = __popcll(pm);
    if (pick) st64(cand + (int64_t)group * m + slot, ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id));
    if (lane >= npk && lane < m) st64(cand + (int64_t)group * m + lane, 0ull);
    if (lane == 0) st32(cand_n + group, (uint32_t)(npk | (nvalid > m ? kGroupDropped : 0)));
}

// One wave's 64-pool group: lanes hold consecutive pools p, `valid` for
// visible ones; keep_best_keys over their scores.
template <class Store64, class Store32>
__device__ __forceinline__ void keep_group_best(float s, bool valid, int p, int group, int m, uint64_t* cand,
                                                int32_t* cand_n, Store64 st64, Store32 st32) {
    keep_best_keys(valid ? f32_key(s) : 0u, valid, (uint32_t)p, __popcll(__ballot(valid)), group, m, cand, cand_n,
                   st64, st32);
}

// ---------------------------------------------------------------- exact top-K of register keys

// Exact top `target` of register keys (0 = absent) under (key descending,
// slot ascending), slot = threadIdx.x * KPT + j, i.e. ties go to the earlier
// slot.  Range bucketing narrows [lo, hi] to the bucket holding rank target
// and stops as soon as that bucket holds at most kBoundCap keys; those are
// ranked exactly by one wave (each compares itself with all of them), so a
// selection usually takes one or two histogram passes.  A bucket of more than
// kBoundCap equal keys is taken in slot order by a block scan.  Returns this
// thread's selected slots as a bitmask (64-bit past 32 keys per thread).
constexpr int kBoundCap = 64;

template <int NT, int KPT>
struct TopSelShared {
    SelShared<NT> S;
    uint32_t mm[2 * NT / 64];
    uint32_t nb;
    uint32_t bkey[kBoundCap];
    uint32_t bslot[kBoundCap];
    uint32_t flag[(NT * KPT + 31) / 32];
};

template <int KPT>
using SlotMask = std::conditional_t<(KPT > 32), uint64_t, uint32_t>;

template <int NT, int KPT>
__device__ __forceinline__ SlotMask<KPT> select_top_slots(const uint32_t (&key)[KPT], uint32_t target,
                                                              TopSelShared<NT, KPT>& T) {
    using Mask = SlotMask<KPT>;
    constexpr int BITS = log2_of<NT>();
    constexpr int FW = (NT * KPT + 31) / 32;
    const int tid = threadIdx.x;
    T.S.hist[0][tid] = 0u;
    T.S.hist[1][tid] = 0u;
    for (int i = tid; i < FW; i += NT) T.flag[i] = 0u;
    if (tid == 0) T.nb = 0u;
    uint32_t lo, hi;
    block_min_max<NT, KPT, uint32_t>(key, T.mm, lo, hi);     // its barriers publish the clears
    uint32_t krem = target, cnt = 0xFFFFFFFFu;
    bool whole = false;
    for (int pass = 0; pass < 4 && lo < hi && cnt > (uint32_t)kBoundCap; ++pass) {
        const int buf = pass & 1;
        const int sh = bit_len<uint32_t>((hi - lo) >> BITS);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t k = key[j];
            if (k >= lo && k <= hi) atomicAdd(&T.S.hist[buf][(k - lo) >> sh], 1u);
        }
        lds_barrier();
        const uint32_t h = T.S.hist[buf][NT - 1 - tid];       // thread order = descending buckets
        T.S.hist[buf ^ 1][tid] = 0u;
        uint32_t total;
        const uint32_t above = block_exclusive_scan<NT>(h, T.S.scan, &total);
        if (above < krem && krem <= above + h) {
            T.S.bin[buf] = NT - 1 - tid;
            T.S.above[buf] = above;
            T.S.cnt[buf] = h;
        }
        lds_barrier();
        krem -= T.S.above[buf];
        cnt = T.S.cnt[buf];
        const uint32_t nlo = lo + (T.S.bin[buf] << sh);
        const uint32_t nhi = nlo + ((1u << sh) - 1u);
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
        if (cnt == krem) {
            whole = true;
            break;
        }
    }
    if (lo == hi && cnt == 0xFFFFFFFFu) {                    // every present key equal (or one key)
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] == lo ? 1u : 0u;
        uint32_t tot;
        block_exclusive_scan<NT>(c, T.S.scan, &tot);
        cnt = tot;
        whole = tot == krem;
    }
    Mask picks = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (key[j] > hi || (whole && key[j] != 0u && key[j] >= lo && key[j] <= hi)) picks |= Mask(1) << j;
    if (whole) return picks;
    if (cnt <= (uint32_t)kBoundCap) {
        // gather the boundary bucket and rank it in one wave
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (key[j] != 0u && key[j] >= lo && key[j] <= hi) {
                const uint32_t e = atomicAdd(&T.nb, 1u);
                T.bkey[e] = key[j];
                T.bslot[e] = (uint32_t)(tid * KPT + j);
            }
        }
        lds_barrier();
        const uint32_t nb = T.nb;
        if ((uint32_t)tid < nb) {
            const uint32_t mk = T.bkey[tid], ms = T.bslot[tid];
            uint32_t rank = 0;
            for (uint32_t i = 0; i < nb; ++i) {
                const uint32_t k = T.bkey[i];
                rank += (k > mk || (k == mk && T.bslot[i] < ms)) ? 1u : 0u;
            }
            if (rank < krem) atomicOr(&T.flag[ms >> 5], 1u << (ms & 31));
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t sl = (uint32_t)(tid * KPT + j);
            if ((T.flag[sl >> 5] >> (sl & 31)) & 1u) picks |= Mask(1) << j;
        }
    } else {
        // more than kBoundCap equal keys (lo == hi): the first krem in slot order
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += (key[j] != 0u && key[j] == lo) ? 1u : 0u;
        uint32_t tot;
        const uint32_t before = block_exclusive_scan<NT>(c, T.S.scan, &tot);
        uint32_t take = krem > before ? min(krem - before, c) : 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (key[j] != 0u && key[j] == lo && take > 0u) {
                picks |= Mask(1) << j;
                --take;
            }
        }
    }
    return picks;
}

// ---------------------------------------------------------------- exact top-K, small workgroups

// The same selection as select_top_slots (same result) for workgroups of a
// few waves holding many keys per thread: every pass has a histogram of its
// own (NB buckets, independent of NT), all cleared up front, and after its
// one barrier every wave finds the rank-target bucket by itself (DPP sums over
// the buckets, read in a bank-conflict-free order), so a pass costs a single
// workgroup barrier; the boundary keys are ranked by every wave too and each
// thread reads its own picks from the resulting ballot.  (With 16 waves the
// repeated per-wave work costs more than it saves, and select_top_slots is
// the faster of the two; a large workgroup here searches and ranks in wave 0
// and hands the result over through LDS.)
constexpr int kSelPasses = 4;

// NB buckets per pass (256, 512 or 1024), independent of the NT threads.
template <int NT, int KPT, int NB = NT>
struct TopSelSmall {
    SelShared<NT> S;                     // block scans (and the fallbacks' state)
    uint32_t hist[kSelPasses][NB];       // one histogram per pass
    uint32_t mm[2 * NT / 64];
    uint32_t nb;
    uint32_t res[4];                     // a pass's bucket (one-wave search) / the boundary picks
    uint32_t bkey[kBoundCap];
    uint32_t bslot[kBoundCap];
};

template <int NT, int KPT, int NB = NT>
__device__ __forceinline__ uint32_t select_top_slots_small(const uint32_t (&key)[KPT], uint32_t target,
                                                     TopSelSmall<NT, KPT, NB>& T) {
    constexpr int BITS = log2_of<NB>();
    constexpr int NW = NT / 64;
    constexpr int PER = NB / 64;                             // buckets per lane in the bucket search
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kSelPasses * NB; i += NT) (&T.hist[0][0])[i] = 0u;
    if (tid == 0) T.nb = 0u;
    // smallest present key and largest key; the barrier also publishes the clears
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (key[j]) lo = min(lo, key[j]);
        hi = max(hi, key[j]);
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        T.mm[2 * w] = lo;
        T.mm[2 * w + 1] = hi;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        lo = min(lo, T.mm[2 * i]);
        hi = max(hi, T.mm[2 * i + 1]);
    }
    uint32_t krem = target, cnt = 0xFFFFFFFFu;
    bool whole = false;
    for (int pass = 0; pass < kSelPasses && lo < hi && cnt > (uint32_t)kBoundCap; ++pass) {
        uint32_t* H = T.hist[pass];
        const int sh = bit_len<uint32_t>((hi - lo) >> BITS);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t k = key[j];
            if (k >= lo && k <= hi) atomicAdd(&H[(k - lo) >> sh], 1u);
        }
        lds_barrier();
        // The rank-krem bucket (d = NB-1-bucket, descending), found by every
        // wave of a small workgroup, or by wave 0 and handed over through LDS
        // in a large one (there the 16-fold repeated search costs more than a
        // second barrier).
        uint32_t d = 0u, above = 0u;
        bool none = false;
        auto search = [&]() {
            // lane l sums d in [l PER, (l+1) PER), read in a rotated order
            // that keeps the 64 lanes on distinct banks
            uint32_t lsum = 0u;
#pragma unroll
            for (int i = 0; i < PER; ++i) lsum += H[NB - 1 - (lane * PER + ((i + lane / (64 / PER)) & (PER - 1)))];
            const uint32_t incl = wave_incl_sum_u32(lsum), excl = incl - lsum;
            const unsigned long long hit = __ballot(excl < krem && krem <= incl);
            if (hit == 0ull) {                               // fewer keys than target: take them all
                none = true;
                return;
            }
            const int L = __ffsll((long long)hit) - 1;
            // walk lane L's buckets (same address in every lane: broadcast reads)
            uint32_t acc = __builtin_amdgcn_readlane(excl, L);
            cnt = 0u;
            bool found = false;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint32_t c = H[NB - 1 - (L * PER + i)];
                if (!found && krem <= acc + c) {
                    found = true;
                    d = (uint32_t)(L * PER + i);
                    above = acc;
                    cnt = c;
                }
                acc += c;
            }
        };
        if constexpr (NW >= 8) {
            if (w == 0) {
                search();
                if (lane == 0) {
                    T.res[0] = d;
                    T.res[1] = above;
                    T.res[2] = cnt;
                    T.res[3] = none ? 1u : 0u;
                }
            }
            lds_barrier();
            d = T.res[0];
            above = T.res[1];
            cnt = T.res[2];
            none = T.res[3] != 0u;
        } else {
            search();
        }
        if (none) {
            whole = true;
            break;
        }
        krem -= above;
        const uint32_t nlo = lo + ((NB - 1 - d) << sh);
        const uint32_t nhi = nlo + ((1u << sh) - 1u);
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
        if (cnt == krem) {
            whole = true;
            break;
        }
    }
    if (lo == hi && cnt == 0xFFFFFFFFu) {                    // every present key equal (or one key)
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] == lo ? 1u : 0u;
        uint32_t tot;
        block_exclusive_scan<NT>(c, T.S.scan, &tot);
        cnt = tot;
        whole = tot == krem;
    }
    uint32_t picks = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (key[j] > hi || (whole && key[j] != 0u && key[j] >= lo && key[j] <= hi)) picks |= 1u << j;
    if (whole) return picks;
    if (cnt <= (uint32_t)kBoundCap) {
        // gather the boundary bucket (a thread's keys take consecutive entries)
        uint32_t mine = 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) mine += (key[j] != 0u && key[j] >= lo && key[j] <= hi) ? 1u : 0u;
        uint32_t e0 = 0u;
        if (mine) {
            e0 = atomicAdd(&T.nb, mine);
            uint32_t e = e0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                if (key[j] != 0u && key[j] >= lo && key[j] <= hi) {
                    T.bkey[e] = key[j];
                    T.bslot[e] = (uint32_t)(tid * KPT + j);
                    ++e;
                }
            }
        }
        lds_barrier();
        // rank the entries (lane i: entry i): every wave of a small
        // workgroup, wave 0 of a large one (handing the picks over in LDS)
        auto rank_entries = [&]() -> unsigned long long {
            const uint32_t nb = T.nb;
            bool pk = false;
            if ((uint32_t)lane < nb) {
                const uint32_t mk = T.bkey[lane], ms = T.bslot[lane];
                uint32_t rank = 0;
                for (uint32_t i = 0; i < nb; ++i) {
                    const uint32_t k = T.bkey[i];
                    rank += (k > mk || (k == mk && T.bslot[i] < ms)) ? 1u : 0u;
                }
                pk = rank < krem;
            }
            return __ballot(pk);
        };
        unsigned long long pm;
        if constexpr (NW >= 8) {
            if (w == 0) {
                pm = rank_entries();
                if (lane == 0) {
                    T.res[0] = (uint32_t)pm;
                    T.res[1] = (uint32_t)(pm >> 32);
                }
            }
            lds_barrier();
            pm = ((unsigned long long)T.res[1] << 32) | T.res[0];
        } else {
            pm = rank_entries();
        }
        uint32_t e = e0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (key[j] != 0u && key[j] >= lo && key[j] <= hi) {
                if ((pm >> e) & 1ull) picks |= 1u << j;
                ++e;
            }
        }
    } else {
        // more than kBoundCap equal keys (lo == hi): the first krem in slot order
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += (key[j] != 0u && key[j] == lo) ? 1u : 0u;
        uint32_t tot;
        const uint32_t before = block_exclusive_scan<NT>(c, T.S.scan, &tot);
        uint32_t take = krem > before ? min(krem - before, c) : 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (key[j] != 0u && key[j] == lo && take > 0u) {
                picks |= 1u << j;
                --take;
            }
        }
    }
    return picks;
}

}  // namespace dsa
