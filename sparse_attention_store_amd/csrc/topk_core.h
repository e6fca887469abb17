// Selection machinery shared by the top-k kernels and the fused decode step:
// query geometry, order-preserving keys, block min/max, range-bucket select
// and order-preserving compaction.  The design notes are at the top of
// topk.hip.
#pragma once

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
template <int NT>
__device__ __forceinline__ void emit_selection(const int32_t* sel, int K, int select_k, int t, int b,
                                               int f, int qp, int n_vis, const Emit& e) {
    const int tid = threadIdx.x;
    if (e.pool_ids) {
        int32_t* out = e.pool_ids + (int64_t)t * select_k;
        for (int i = tid; i < select_k; i += NT) out[i] = i < K ? (sel ? sel[i] : i) : -1;
    }
    if (e.indices) {
        const int64_t rb = e.row_base[b];
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
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const KT a = shfl_xor_k(mn, o), c = shfl_xor_k(mx, o);
        mn = a < mn ? a : mn;
        mx = c > mx ? c : mx;
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

template <int NT>
constexpr int log2_of() { return NT == 256 ? 8 : (NT == 512 ? 9 : 10); }

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

}  // namespace dsa
