// topk_select: per query, the K = min(select_k, n_vis) best pools by
// (score descending, pool id ascending), emitted in ascending id order and
// padded with -1 ([Ref] Functions: topk_pools; [Flash] Stream C:
// indexer_topk512).  Scores are mapped to order-preserving uint32 keys.
//
// Two paths:
//  * rows: one 1024-thread workgroup per query row, the whole row of keys in
//    LDS.  The K-th largest key is found by range bucketing: each pass
//    histograms the keys inside [lo, hi] into 2048 equal-width buckets
//    (integer arithmetic on the key), keeps the bucket that holds rank K and
//    narrows [lo, hi] to it; a 32-bit key range closes in at most 3 passes.
//    A scan in id order then emits every key above the threshold and the
//    first `need` keys equal to it, which is exactly the tie rule.
//  * long: rows too long for LDS (decode at 262k..1M context) are split over
//    many workgroups.  Launch 1 builds a 4096-bin histogram of the key's top
//    12 bits per row (LDS histogram, then one global add per non-empty bin);
//    the last workgroup of the row (atomic ticket) finds the bin holding rank
//    K.  Launch 2 sends keys above that bin to a "sure" list and keys inside
//    it to a candidate list of 64-bit (key, ~id) composites; the last
//    workgroup selects the best candidates exactly (composites are unique, so
//    no tie remains), bitonic-sorts the K ids and writes them.  Counters,
//    histograms and tickets are cleared by the workgroup that consumed them,
//    so the workspace stays zero-filled between calls.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kRowNT = 1024;
constexpr int kRowBins = 2048;
constexpr int kLongNT = 256;
constexpr int kLongChunk = 4096;          // keys per workgroup (long path)
constexpr int kLongBins = 4096;           // level-1 bins: key >> 20
constexpr int kLongMaxK = 1024;           // select_k limit of the long path
constexpr int kCandLds = 4096;            // candidates held in LDS by the finishing workgroup

struct TopkRowHdr {                       // 64 bytes per query row
    uint32_t hist_done, filt_done, n_sure, n_cand, thr_bin, above, pad[10];
};

__device__ __forceinline__ int n_visible(const int32_t* first_valid, const int32_t* q_seq,
                                         const int32_t* q_pos, int t) {
    const int b = q_seq[t];
    const int f = first_valid[b];
    const int qp = q_pos[t];
    return qp >= f ? (qp - f + 1) >> 2 : 0;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- rows path

template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* sh) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = sh[0];
    for (int w = 1; w < NT / 64; ++w) r = min(r, sh[w]);
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = sh[0];
    for (int w = 1; w < NT / 64; ++w) r = max(r, sh[w]);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kRowNT) void k_topk_rows(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int select_k,
    int32_t* __restrict__ pool_ids) {
    extern __shared__ uint32_t keys[];
    __shared__ uint32_t hist[kRowBins];
    __shared__ uint32_t scan_sh[kRowNT / 64 + 1];
    __shared__ uint32_t s_bin, s_above;

    const int t = blockIdx.x, tid = threadIdx.x;
    const int n = min(n_visible(first_valid, q_seq, q_pos, t), stride);
    int32_t* out = pool_ids + (int64_t)t * select_k;
    if (n <= select_k) {                                  // every visible pool is selected
        for (int i = tid; i < select_k; i += kRowNT) out[i] = i < n ? i : -1;
        return;
    }
    const float* row = scores + (int64_t)t * stride;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = tid; i < n; i += kRowNT) {
        const uint32_t k = f32_key(row[i]);
        keys[i] = k;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
    }
    kmin = block_min_u32<kRowNT>(kmin, scan_sh);
    kmax = block_max_u32<kRowNT>(kmax, scan_sh);

    uint32_t lo = kmin, hi = kmax, krem = (uint32_t)select_k;
    // A 32-bit range closes in 3 passes; the cap only bounds the loop.
    for (int pass = 0; pass < 6 && lo < hi; ++pass) {
        const uint64_t range = (uint64_t)(hi - lo) + 1u;
        for (int b = tid; b < kRowBins; b += kRowNT) hist[b] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += kRowNT) {
            const uint32_t k = keys[i];
            if (k >= lo && k <= hi)
                atomicAdd(&hist[(uint32_t)(((uint64_t)(k - lo) * kRowBins) / range)], 1u);
        }
        __syncthreads();
        // Thread j owns buckets kRowBins-1-2j and kRowBins-2-2j (scanned from the top).
        const int b0 = kRowBins - 1 - 2 * tid, b1 = b0 - 1;
        const uint32_t h0 = hist[b0], h1 = hist[b1];
        uint32_t total;
        const uint32_t above = block_exclusive_scan<kRowNT>(h0 + h1, scan_sh, &total);
        if (above < krem && krem <= above + h0) { s_bin = b0; s_above = above; }
        else if (above + h0 < krem && krem <= above + h0 + h1) { s_bin = b1; s_above = above + h0; }
        __syncthreads();
        const uint64_t bin = s_bin;
        krem -= s_above;
        const uint32_t nlo = lo + (uint32_t)((bin * range + kRowBins - 1) / kRowBins);
        const uint32_t nhi = lo + (uint32_t)(((bin + 1) * range + kRowBins - 1) / kRowBins) - 1u;
        lo = nlo;
        hi = nhi;
        __syncthreads();
    }
    const uint32_t tau = lo, need_eq = krem;

    // Emit in id order: keys > tau, plus the first need_eq keys == tau.
    const int per = (n + kRowNT - 1) / kRowNT;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    uint32_t gt = 0, eq = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        gt += k > tau;
        eq += k == tau;
    }
    uint32_t total;
    const uint32_t eq_base = block_exclusive_scan<kRowNT>(eq, scan_sh, &total);
    uint32_t take = need_eq > eq_base ? min(need_eq - eq_base, eq) : 0u;
    const uint32_t pos0 = block_exclusive_scan<kRowNT>(gt + take, scan_sh, &total);
    uint32_t pos = pos0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        const bool pick = k > tau || (k == tau && take > 0);
        if (k == tau && pick) --take;
        if (pick && pos < (uint32_t)select_k) out[pos] = i;
        pos += pick;
    }
}

// ---------------------------------------------------------------- long path

struct LongWs {
    TopkRowHdr* hdr;
    uint32_t* hist;     // [T][kLongBins]
    int32_t* sure;      // [T][select_k]
    uint64_t* cand;     // [T][stride]
};

__device__ __forceinline__ LongWs long_ws(void* ws, int T, int select_k, int stride) {
    char* p = reinterpret_cast<char*>(ws);
    LongWs w;
    w.hdr = reinterpret_cast<TopkRowHdr*>(p);
    p += ((size_t)T * sizeof(TopkRowHdr) + 255) & ~(size_t)255;
    w.hist = reinterpret_cast<uint32_t*>(p);
    p += ((size_t)T * kLongBins * 4 + 255) & ~(size_t)255;
    w.sure = reinterpret_cast<int32_t*>(p);
    p += ((size_t)T * select_k * 4 + 255) & ~(size_t)255;
    w.cand = reinterpret_cast<uint64_t*>(p);
    return w;
}

__global__ __launch_bounds__(kLongNT) void k_topk_long_hist(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int select_k, int T,
    void* ws, int groups) {
    __shared__ uint32_t h[kLongBins];
    __shared__ uint32_t scan_sh[kLongNT / 64 + 1];
    __shared__ int s_last;
    const int t = blockIdx.y, tid = threadIdx.x;
    const int n = min(n_visible(first_valid, q_seq, q_pos, t), stride);
    if (n <= select_k) return;
    LongWs w = long_ws(ws, T, select_k, stride);
    TopkRowHdr* hdr = w.hdr + t;
    uint32_t* gh = w.hist + (size_t)t * kLongBins;

    for (int b = tid; b < kLongBins; b += kLongNT) h[b] = 0u;
    __syncthreads();
    const float* row = scores + (int64_t)t * stride;
    const int i0 = blockIdx.x * kLongChunk, i1 = min(i0 + kLongChunk, n);
    for (int i = i0 + tid; i < i1; i += kLongNT) atomicAdd(&h[f32_key(row[i]) >> 20], 1u);
    __syncthreads();
    for (int b = tid; b < kLongBins; b += kLongNT)
        if (h[b]) atomicAdd(&gh[b], h[b]);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&hdr->hist_done, 1u) == (uint32_t)(groups - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Last workgroup of the row: find the bin holding rank K, scanning from the top.
    constexpr int PER = kLongBins / kLongNT;               // 16 bins per thread
    uint32_t loc[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        loc[j] = ld_agent(&gh[kLongBins - 1 - (tid * PER + j)]);
        sum += loc[j];
    }
    uint32_t total;
    uint32_t above = block_exclusive_scan<kLongNT>(sum, scan_sh, &total);
    const uint32_t K = (uint32_t)select_k;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (above < K && K <= above + loc[j]) {
            hdr->thr_bin = (uint32_t)(kLongBins - 1 - (tid * PER + j));
            hdr->above = above;
        }
        above += loc[j];
    }
    for (int b = tid; b < kLongBins; b += kLongNT) gh[b] = 0u;
    if (tid == 0) hdr->hist_done = 0u;
}

// Rank-r threshold among n unique 64-bit composites: returns the r-th largest.
template <int NT>
__device__ uint64_t select_u64_rank(const uint64_t* src, uint32_t n, uint32_t r, uint32_t* hist,
                                    uint32_t* scan_sh, uint64_t* s_lo, uint64_t* s_hi,
                                    uint32_t* s_krem) {
    constexpr int NB = 2048;
    const int tid = threadIdx.x;
    uint64_t lmin = ~0ull, lmax = 0ull;
    for (uint32_t i = tid; i < n; i += NT) {
        const uint64_t v = src[i];
        lmin = v < lmin ? v : lmin;
        lmax = v > lmax ? v : lmax;
    }
    if (tid == 0) { *s_lo = ~0ull; *s_hi = 0ull; *s_krem = r; }
    __syncthreads();
    atomicMin((unsigned long long*)s_lo, (unsigned long long)lmin);
    atomicMax((unsigned long long*)s_hi, (unsigned long long)lmax);
    __syncthreads();
    uint64_t lo = *s_lo, hi = *s_hi;
    uint32_t krem = r;
    __shared__ uint32_t s_bin, s_above;
    // A 52-bit range closes in 5 passes; the cap only bounds the loop.
    for (int pass = 0; pass < 8 && lo < hi; ++pass) {
        const uint64_t range = hi - lo + 1u;                // < 2^52 (keys share their top 12 bits)
        for (int b = tid; b < NB; b += NT) hist[b] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < n; i += NT) {
            const uint64_t v = src[i];
            if (v >= lo && v <= hi) atomicAdd(&hist[(uint32_t)(((v - lo) * NB) / range)], 1u);
        }
        __syncthreads();
        constexpr int PER = NB / NT;
        uint32_t loc[PER];
        uint32_t sum = 0;
        for (int j = 0; j < PER; ++j) {
            loc[j] = hist[NB - 1 - (tid * PER + j)];
            sum += loc[j];
        }
        uint32_t total;
        uint32_t above = block_exclusive_scan<NT>(sum, scan_sh, &total);
        for (int j = 0; j < PER; ++j) {
            if (above < krem && krem <= above + loc[j]) {
                s_bin = (uint32_t)(NB - 1 - (tid * PER + j));
                s_above = above;
            }
            above += loc[j];
        }
        __syncthreads();
        const uint64_t bin = s_bin;
        krem -= s_above;
        const uint64_t nlo = lo + (bin * range + NB - 1) / NB;
        const uint64_t nhi = lo + ((bin + 1) * range + NB - 1) / NB - 1u;
        lo = nlo;
        hi = nhi;
        __syncthreads();
    }
    return lo;
}

__global__ __launch_bounds__(kLongNT) void k_topk_long_filter(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ first_valid,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int select_k, int T,
    void* ws, int groups, int32_t* __restrict__ pool_ids) {
    __shared__ uint64_t l_cand[kCandLds];
    __shared__ int32_t l_sel[kLongMaxK];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t scan_sh[kLongNT / 64 + 1];
    __shared__ uint32_t l_ns, l_nc, s_sbase, s_cbase, s_krem;
    __shared__ uint64_t s_lo, s_hi;
    __shared__ int s_last;

    const int t = blockIdx.y, tid = threadIdx.x;
    const int n = min(n_visible(first_valid, q_seq, q_pos, t), stride);
    int32_t* out = pool_ids + (int64_t)t * select_k;
    if (n <= select_k) {
        if (blockIdx.x == 0)
            for (int i = tid; i < select_k; i += kLongNT) out[i] = i < n ? i : -1;
        return;
    }
    LongWs w = long_ws(ws, T, select_k, stride);
    TopkRowHdr* hdr = w.hdr + t;
    int32_t* gsure = w.sure + (size_t)t * select_k;
    uint64_t* gcand = w.cand + (size_t)t * stride;
    const uint32_t thr = hdr->thr_bin;

    if (tid == 0) { l_ns = 0u; l_nc = 0u; }
    __syncthreads();
    const float* row = scores + (int64_t)t * stride;
    const int i0 = blockIdx.x * kLongChunk, i1 = min(i0 + kLongChunk, n);
    for (int i = i0 + tid; i < i1; i += kLongNT) {
        const uint32_t k = f32_key(row[i]);
        const uint32_t bin = k >> 20;
        if (bin > thr) {
            const uint32_t j = atomicAdd(&l_ns, 1u);       // < select_k per row in total
            if (j < (uint32_t)kLongMaxK) l_sel[j] = i;
        } else if (bin == thr) {
            const uint32_t j = atomicAdd(&l_nc, 1u);       // <= kLongChunk per workgroup
            if (j < (uint32_t)kCandLds) l_cand[j] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
        }
    }
    __syncthreads();
    if (tid == 0) {
        s_sbase = l_ns ? atomicAdd(&hdr->n_sure, l_ns) : 0u;
        s_cbase = l_nc ? atomicAdd(&hdr->n_cand, l_nc) : 0u;
    }
    __syncthreads();
    for (uint32_t j = tid; j < l_ns; j += kLongNT)
        if (s_sbase + j < (uint32_t)select_k) gsure[s_sbase + j] = l_sel[j];
    for (uint32_t j = tid; j < l_nc; j += kLongNT)
        if (s_cbase + j < (uint32_t)stride) gcand[s_cbase + j] = l_cand[j];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&hdr->filt_done, 1u) == (uint32_t)(groups - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Last workgroup: exact selection among the threshold-bin candidates.
    const uint32_t ns = min(ld_agent(&hdr->n_sure), (uint32_t)select_k);
    const uint32_t nc = min(ld_agent(&hdr->n_cand), (uint32_t)stride);
    const uint32_t need = (uint32_t)select_k - ns;
    const uint64_t* src = gcand;
    if (nc <= (uint32_t)kCandLds) {
        for (uint32_t j = tid; j < nc; j += kLongNT) l_cand[j] = __hip_atomic_load(&gcand[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        src = l_cand;
        __syncthreads();
    }
    const uint64_t tau = select_u64_rank<kLongNT>(src, nc, need, hist, scan_sh, &s_lo, &s_hi, &s_krem);
    for (uint32_t j = tid; j < ns; j += kLongNT) l_sel[j] = __hip_atomic_load(&gsure[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) l_ns = ns;
    __syncthreads();
    for (uint32_t j = tid; j < nc; j += kLongNT) {
        const uint64_t v = src[j];
        if (v >= tau) {
            const uint32_t s2 = atomicAdd(&l_ns, 1u);
            if (s2 < (uint32_t)select_k) l_sel[s2] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
        }
    }
    __syncthreads();
    int P = 1;
    while (P < select_k) P <<= 1;
    for (int j = select_k + tid; j < P; j += kLongNT) l_sel[j] = 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < P; i += kLongNT) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const int a = l_sel[i], b = l_sel[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) { l_sel[i] = b; l_sel[ixj] = a; }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < select_k; i += kLongNT) out[i] = l_sel[i];
    if (tid == 0) {
        hdr->n_sure = 0u;
        hdr->n_cand = 0u;
        hdr->filt_done = 0u;
    }
}

}  // namespace dsa

namespace dsa_host {

static size_t rows_lds_bytes(int32_t stride) { return (size_t)stride * 4; }

static bool use_rows_path(const dsa_dims& d, int32_t stride) {
    const size_t static_lds = dsa::kRowBins * 4 + 256;
    return rows_lds_bytes(stride) + static_lds <= device_info().max_lds_per_block ||
           d.index_topk / d.kpool > dsa::kLongMaxK;
}

static size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t topk_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride) {
    if (T <= 0 || stride <= 0 || use_rows_path(d, stride)) return 0;
    const size_t sk = (size_t)(d.index_topk / d.kpool);
    return r256((size_t)T * sizeof(dsa::TopkRowHdr)) + r256((size_t)T * dsa::kLongBins * 4) +
           r256((size_t)T * sk * 4) + r256((size_t)T * stride * 8);
}

hipError_t launch_topk(const dsa_dims& d, const float* scores, int32_t stride, const dsa_seqs& seqs,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                       void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int sk = d.index_topk / d.kpool;
    if (use_rows_path(d, stride)) {
        const size_t lds = rows_lds_bytes(stride);
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dsa::k_topk_rows),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(dsa::k_topk_rows, dim3((unsigned)T), dim3(dsa::kRowNT), lds, s, scores,
                           stride, seqs.first_valid, q_seq, q_pos, sk, pool_ids);
        return hipGetLastError();
    }
    const int groups = (int)cdiv(stride, dsa::kLongChunk);
    dim3 grid((unsigned)groups, (unsigned)T);
    hipLaunchKernelGGL(dsa::k_topk_long_hist, grid, dim3(dsa::kLongNT), 0, s, scores, stride,
                       seqs.first_valid, q_seq, q_pos, sk, (int)T, ws, groups);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dsa::k_topk_long_filter, grid, dim3(dsa::kLongNT), 0, s, scores, stride,
                       seqs.first_valid, q_seq, q_pos, sk, (int)T, ws, groups, pool_ids);
    return hipGetLastError();
}

}  // namespace dsa_host
