// topk_select: per query, the K = min(select_k, n_vis) best pools by
// (score descending, pool id ascending), emitted in ascending id order and
// padded with -1 ([Ref] Functions: topk_pools; [Flash] Stream C:
// indexer_topk512).  Optionally the same launches also write the expanded
// index list ([Ref] Functions: expand_selection).
//
// Two stages, no cross-workgroup atomics and no state kept between calls:
//  A. Each query row is cut into chunks of 4096 pools.  One 256-thread
//     workgroup per chunk selects the chunk's best min(select_k, chunk) pools
//     under the same order and writes them, in ascending id order, as 64-bit
//     composites (key << 32 | ~id), where key is the order-preserving uint32
//     image of the fp32 score (-0 mapped to +0).  Every member of the row's
//     top-K is in its chunk's top-K under this total order, so the union of
//     the chunk lists contains the answer.
//  B. One 1024-thread workgroup per row selects the best K of that union (at
//     most 64 chunks x select_k, held in registers).  The chunk lists are in
//     ascending id order, so the same 32-bit key selection with ties taken in
//     list order applies the tie rule, and a scan-based compaction emits the
//     ids sorted.
// Both stages find the K-th largest key by range bucketing in LDS: each pass
// histograms the keys inside [lo, hi] into one bucket per thread, of width
// 2^sh (the key offset shifted right), keeps the bucket that holds rank K and
// narrows [lo, hi] to it, until that bucket is taken whole or (stage A) one key
// value is left, whose first `need` occurrences in id order are taken -- the
// tie rule.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kChunkKeys = 4096;            // pools per stage-A workgroup
constexpr int kANT = 256, kAKPT = kChunkKeys / kANT;
constexpr int kBNT = 1024;
constexpr int kMaxK = 1024;                 // select_k limit
constexpr int kMaxCand = 32 * kBNT;         // stage-B capacity (chunks x select_k)

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

// ---------------------------------------------------------------- stage A

__global__ __launch_bounds__(kANT) void k_topk_chunks(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int select_k, int nchunks,
    uint64_t* __restrict__ cand, int32_t* __restrict__ cand_n) {
    __shared__ SelShared<kANT> S;
    __shared__ uint32_t mm_sh[2 * kANT / 64];
    const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int n = min(n_vis, stride);
    if (n <= select_k) return;                               // stage B selects every pool
    const int c0 = c * kChunkKeys;
    const int cn = max(0, min(n - c0, kChunkKeys));          // keys in this chunk
    uint64_t* out = cand + ((int64_t)t * nchunks + c) * select_k;
    const float* row = scores + (int64_t)t * stride + c0;
    if (cn <= select_k) {                                    // the whole chunk is a candidate set
        for (int i = tid; i < cn; i += kANT)
            out[i] = ((uint64_t)f32_key(row[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(c0 + i));
        if (tid == 0) cand_n[t * nchunks + c] = cn;
        return;
    }
    // Keys [c0 + tid*16, +16); absent keys are 0, below every real key.
    const int i0 = tid * kAKPT;
    uint32_t key[kAKPT];
    const bool vec = ((stride & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
    if (vec && i0 + kAKPT <= cn) {
#pragma unroll
        for (int q = 0; q < kAKPT / 4; ++q) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(row + i0 + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) key[4 * q + e] = f32_key(v[e]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kAKPT; ++j) key[j] = (i0 + j < cn) ? f32_key(row[i0 + j]) : 0u;
    }
    uint32_t lo, hi, krem;
    bool whole;
    bucket_select<kANT, kAKPT, uint32_t>(key, (uint32_t)select_k, S, mm_sh, lo, hi, krem, whole);
    uint32_t take;
    uint32_t pos = compaction_slot<kANT, kAKPT, uint32_t>(key, lo, hi, krem, whole, S, take);
#pragma unroll
    for (int j = 0; j < kAKPT; ++j) {
        const uint32_t k = key[j];
        const bool inr = k >= lo && k <= hi;
        const bool pick = k > hi || (inr && take > 0);
        take -= (inr && take > 0) ? 1u : 0u;
        if (pick && pos < (uint32_t)select_k)
            out[pos] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(c0 + i0 + j));
        pos += pick;
    }
    if (tid == 0) cand_n[t * nchunks + c] = select_k;
}

// ---------------------------------------------------------------- stage B

template <int KPT>
__global__ __launch_bounds__(kBNT) void k_topk_merge(
    const int32_t* __restrict__ first_valid, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int stride, int select_k, int nchunks,
    const uint64_t* __restrict__ cand, const int32_t* __restrict__ cand_n, Emit e) {
    __shared__ SelShared<kBNT> S;
    __shared__ uint32_t mm_sh[2 * kBNT / 64];
    __shared__ int32_t sel[kMaxK];
    const int t = blockIdx.x, tid = threadIdx.x;
    int b, f, qp, n_vis;
    query_geom(first_valid, q_seq, q_pos, t, b, f, qp, n_vis);
    const int n = min(n_vis, stride);
    if (n <= select_k) {                                     // every visible pool is selected
        emit_selection<kBNT>(nullptr, n, select_k, t, b, f, qp, n_vis, e);
        return;
    }
    // Candidate slot s = chunk * select_k + i; slots past a chunk's count are absent
    // (key 0).  Slots are in ascending pool-id order, so among equal keys the
    // first ones in slot order have the lowest ids: the 32-bit key alone plus
    // the in-order tie step reproduces the rule.
    const int used = (n + kChunkKeys - 1) / kChunkKeys;      // chunks stage A wrote for this row
    const uint64_t* cr = cand + (int64_t)t * nchunks * select_k;
    const int M = used * select_k;
    const int s0 = tid * KPT;
    uint32_t key[KPT];
    int32_t id[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int s = s0 + j;
        key[j] = 0u;
        id[j] = 0;
        if (s < M) {
            const int ch = s / select_k;
            if (s - ch * select_k < cand_n[t * nchunks + ch]) {
                const uint64_t v = cr[s];
                key[j] = (uint32_t)(v >> 32);
                id[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
            }
        }
    }
    uint32_t lo, hi, krem;
    bool whole;
    bucket_select<kBNT, KPT, uint32_t>(key, (uint32_t)select_k, S, mm_sh, lo, hi, krem, whole);
    uint32_t take;
    uint32_t pos = compaction_slot<kBNT, KPT, uint32_t>(key, lo, hi, krem, whole, S, take);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t k = key[j];
        const bool inr = k >= lo && k <= hi;
        const bool pick = k > hi || (inr && take > 0);
        take -= (inr && take > 0) ? 1u : 0u;
        if (pick && pos < (uint32_t)kMaxK) sel[pos] = id[j];
        pos += pick;
    }
    lds_barrier();
    emit_selection<kBNT>(sel, select_k, select_k, t, b, f, qp, n_vis, e);
}

}  // namespace dsa

namespace dsa_host {

static int topk_chunks(int32_t stride) { return (int)cdiv(stride, dsa::kChunkKeys); }

static size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }

bool topk_supported(const dsa_dims& d, int32_t stride) {
    const int sk = d.index_topk / d.kpool;
    return sk <= dsa::kMaxK && (int64_t)topk_chunks(stride) * sk <= dsa::kMaxCand;
}

size_t topk_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride) {
    if (T <= 0 || stride <= 0) return 0;
    const size_t sk = (size_t)(d.index_topk / d.kpool);
    const size_t nc = (size_t)topk_chunks(stride);
    return r256((size_t)T * nc * sk * 8) + r256((size_t)T * nc * 4);
}

hipError_t launch_topk(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                       int32_t* indices, void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int sk = d.index_topk / d.kpool;
    const int nc = topk_chunks(stride);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
    int32_t* cand_n = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + r256((size_t)T * nc * sk * 8));
    const dsa::Emit e{pool_ids, indices, seqs.row_base, d.out_width};
    hipLaunchKernelGGL(dsa::k_topk_chunks, dim3((unsigned)nc, (unsigned)T), dim3(dsa::kANT), 0, s, scores,
                       stride, seqs.first_valid, q_seq, q_pos, sk, nc, cand, cand_n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int kpt = (int)cdiv((int64_t)nc * sk, dsa::kBNT);
#define DSA_MERGE(KPT)                                                                                    \
    hipLaunchKernelGGL((dsa::k_topk_merge<KPT>), dim3((unsigned)T), dim3(dsa::kBNT), 0, s, seqs.first_valid, \
                       q_seq, q_pos, stride, sk, nc, cand, cand_n, e)
    if (kpt <= 1) DSA_MERGE(1);
    else if (kpt <= 2) DSA_MERGE(2);
    else if (kpt <= 4) DSA_MERGE(4);
    else if (kpt <= 8) DSA_MERGE(8);
    else if (kpt <= 16) DSA_MERGE(16);
    else DSA_MERGE(32);
#undef DSA_MERGE
    return hipGetLastError();
}

}  // namespace dsa_host
