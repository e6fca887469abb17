// decode_step: the decode-step chain index_scores -> topk_select ->
// expand_selection -> sparse_mla (-> combine) in one persistent launch
// ([Ref] Functions: index_scores, topk_pools, expand_selection,
// mla_masked_attention; [Kernels] Included: split-KV decode).
//
// Every workgroup (one per CU, 256 threads) claims tasks from one queue.  For
// the query of rank r (queries ranked by decreasing length) the queue holds:
//   * scoring tasks: 512 pools each, two 64-pool groups per wave.  A wave
//     loads its groups one task ahead straight into MFMA registers and scores
//     each with the same per-wave group code as the standalone decode scoring
//     kernel (so the two agree bit for bit); each group then keeps its best m
//     pools by (score desc, id asc): the m-th largest key is found with 32
//     ballot-and-popcount steps, no LDS;
//   * one selection task (sparse queries only): the best K of the group
//     lists, checked against the same certificate as the standalone top-k (a
//     group that dropped pools must not have all m kept ones selected), with
//     the exact streaming radix select over the query's scores as the
//     fallback;
//   * attention tasks: one per (split of 128 list positions, 16 heads).
//     Dense queries (n_vis <= select_k) need no selection;
//   * combine tasks (when a query has more than one split): 4 heads each,
//     merging the split partials in split order.
// Queue order: the tiles of rank 0, the tiles of rank 1, the selection of
// rank 0, the tiles of rank 2, the selection of rank 1, ... so a selection is
// claimed once its query's tiles have been claimed a while; then every
// attention task, then every combine task.  Attention and combine tasks thus
// never hold a CU while scoring work is left.  A task only ever waits for
// tasks earlier in the queue, which were claimed by running workgroups, so
// the launch always drains whatever the number of resident workgroups; every
// wait is bounded (a timeout sets the error word and carries on).  Only a
// scoring task claims its successor early (to prefetch it), so a long task
// never holds a claimed tile back.
//
// Data handed between workgroups of the launch (scores, group lists, the
// selection, attention partials) is written with relaxed agent-scope atomic
// stores and read with relaxed agent-scope atomic loads: these bypass the
// per-XCD L2, which is not coherent across XCDs, so no cache write-back or
// invalidate is needed.  A producer waits for its own stores to complete
// (s_waitcnt vmcnt(0)), synchronises its workgroup, then bumps a counter; a
// consumer polls the counter, synchronises, then loads.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "mla_core.h"
#include "scores_core.h"
#include "topk_core.h"

namespace dsa {

constexpr int kStepMaxT = 64;
constexpr int kSTile = 512;              // pools per scoring task (two 256-pool halves)
constexpr int kSGroup = kGroupPools;
constexpr int kStepMaxGroups = kMaxGroups;
constexpr int kStepCandCap = kGroupCandCap;
constexpr int kStepNT = 256;
constexpr int kStepKPT = kStepCandCap / kStepNT;
constexpr int kStepMaxK = kGroupMaxK;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kCombHeads = 4;            // heads per combine task

struct StepCounters {                    // zero between launches (the last workgroup out resets them)
    uint32_t queue;
    uint32_t exited;
    uint32_t error;
    uint32_t pad;
    uint32_t tiles_done[kStepMaxT];
    uint32_t sel_ready[kStepMaxT];
    uint32_t splits_done[kStepMaxT];
};

struct StepArgs {
    int T, H, W, select_k, stride, splits, grid;
    float scale_log2;
    const uint16_t* q_idx;
    const float* w;
    const uint16_t* pools;
    const int32_t* first_valid;
    const int64_t* pool_base;
    const int64_t* row_base;
    const int32_t* q_seq;
    const int32_t* q_pos;
    const uint16_t* q;
    const uint8_t* cache;
    int row_bytes;
    void* out;
    int out_f32;
    float* lse;
    int32_t* pool_ids;
    int32_t* indices;
    StepCounters* ctr;
    float* scores;
    uint64_t* cand;
    int32_t* cand_n;
    int32_t* sel;
    float* part_o;
    MlaPartial* part_ml;
};

// ---------------------------------------------------------------- coherent access

__device__ __forceinline__ void st_coh32(void* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(void* p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh32(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte agent-coherent loads: a raw buffer load with the sc1 cache policy
// (the bit the relaxed agent-scope atomic loads above carry).
constexpr int kCachePolicySC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base, uint32_t bytes) {
    return buffer_rsrc(base, bytes);
}
__device__ __forceinline__ u32x4 ld_coh128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicySC1);
}

// This thread's outstanding memory operations are complete (stores
// acknowledged), and the compiler moves no memory access across.
__device__ __forceinline__ void drain_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Publish: every thread's stores so far are complete, then one counter bump
// (no return value awaited).
__device__ __forceinline__ void publish(uint32_t* counter) {
    drain_memory();
    lds_barrier();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until *counter >= target (thread 0 polls), then synchronise.
__device__ __forceinline__ void wait_counter(const uint32_t* counter, uint32_t target, uint32_t* err) {
    if (threadIdx.x == 0) {
        uint32_t spins = 0;
        while (ld_coh32(counter) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    lds_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- shared memory

struct StepPlan {
    int order[kStepMaxT];        // queries by decreasing tile count (ties: lower index first)
    int nvis[kStepMaxT];
    int first[kStepMaxT];        // first_valid of the query's sequence
    int tail[kStepMaxT];
    int ntiles[kStepMaxT];
    int64_t pbase[kStepMaxT];
    int64_t rbase[kStepMaxT];
    int seg[4 * kStepMaxT + 3];         // first task of each segment
    uint8_t seg_stage[4 * kStepMaxT + 2];
    uint8_t seg_rank[4 * kStepMaxT + 2];
    int n_seg, n_total;
    uint32_t bcast;
    int task;
};

struct StepSelSmem {
    TopSelSmall<kStepNT, kStepKPT, 1024> T;
    int32_t sel[kStepMaxK];
    uint32_t gpicked[kStepMaxGroups];
    uint32_t gcount[kStepMaxGroups];
    int fail;
};

struct StepCombSmem {
    float wgt[kCombHeads][kMaxSplits];
    float M[kCombHeads], L[kCombHeads];
};

union StepSmem {
    StepSelSmem sel;
    MlaRowsSmem mla;
    StepCombSmem comb;
};

// ---------------------------------------------------------------- selection (continuation)

// Exact top-K straight from the query's scores (coherent loads), as
// topk_stream_exact does, for NT = 256.  Writes K ascending ids to sel.
__device__ void step_stream_exact(const float* row, int n, int K, SelShared<kStepNT>& S, int32_t* sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K, total;
    for (int d = 3; d >= 0; --d) {
        S.hist[0][tid] = 0u;
        lds_barrier();
        for (int i = tid; i < n; i += kStepNT) {
            const uint32_t k = f32_key(__uint_as_float(ld_coh32(row + i)));
            if ((k & mask) == prefix) atomicAdd(&S.hist[0][(k >> (8 * d)) & 0xFFu], 1u);
        }
        lds_barrier();
        const uint32_t h = S.hist[0][255 - tid];
        const uint32_t above = block_exclusive_scan<kStepNT>(h, S.scan, &total);
        if (above < need && need <= above + h) {
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
    for (int i0 = 0; i0 < n; i0 += kStepNT) {
        const int i = i0 + tid;
        const uint32_t k = i < n ? f32_key(__uint_as_float(ld_coh32(row + i))) : 0u;
        const uint32_t gt = (i < n && k > prefix) ? 1u : 0u;
        const uint32_t eq = (i < n && k == prefix) ? 1u : 0u;
        uint32_t eq_tot, pick_tot;
        const uint32_t eq_rank = eq_base + block_exclusive_scan<kStepNT>(eq, S.scan, &eq_tot);
        const uint32_t pick = gt | ((eq && eq_rank < need) ? 1u : 0u);
        const uint32_t pos = out_base + block_exclusive_scan<kStepNT>(pick, S.scan, &pick_tot);
        if (pick && pos < (uint32_t)kStepMaxK) sel[pos] = i;
        out_base += pick_tot;
        eq_base += eq_tot;
    }
}

// The selection of query t from its group lists; publishes sel[t][0..K).
__device__ void step_select(const StepArgs& a, StepSelSmem& sm, StepPlan& plan, int t) {
    const int tid = threadIdx.x;
    const int n = plan.nvis[t], K = a.select_k;
    const int groups = (n + kSGroup - 1) / kSGroup;
    const int m = group_quota<true>(K, n);
    const int msh = __ffs(m) - 1;
    const int M = groups * m;
    const int32_t* cn = a.cand_n + (int64_t)t * kStepMaxGroups;
    const uint64_t* cr = a.cand + (int64_t)t * kStepCandCap;
    // Every load is issued at once: the group counts (kept in LDS) and this
    // thread's kStepKPT slots, all inside the buffer, masked afterwards.
    const int s0 = tid * kStepKPT;
    uint32_t gc[kStepMaxGroups / kStepNT];
#pragma unroll
    for (int k = 0; k < kStepMaxGroups / kStepNT; ++k) {
        const int gi = tid + k * kStepNT;
        gc[k] = gi < groups ? ld_coh32(cn + gi) : 0u;
    }
    uint64_t raw[kStepKPT];
    {
        const __amdgpu_buffer_rsrc_t rs = coh_rsrc(cr, kStepCandCap * 8);
#pragma unroll
        for (int j = 0; j < kStepKPT; j += 2) {
            const u32x4 v = ld_coh128(rs, (uint32_t)(s0 + j) * 8u);
            raw[j] = ((uint64_t)v[1] << 32) | v[0];
            raw[j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    }
#pragma unroll
    for (int k = 0; k < kStepMaxGroups / kStepNT; ++k) {
        sm.gcount[tid + k * kStepNT] = gc[k];
        sm.gpicked[tid + k * kStepNT] = 0u;
    }
    if (tid == 0) sm.fail = 0;
    lds_barrier();
    uint32_t key[kStepKPT];
    int32_t id[kStepKPT];
#pragma unroll
    for (int j = 0; j < kStepKPT; ++j) {
        const int s = s0 + j;
        const bool ok = s < M && (s & (m - 1)) < (int)(sm.gcount[s >> msh] & (kGroupDropped - 1));
        key[j] = ok ? (uint32_t)(raw[j] >> 32) : 0u;
        id[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)raw[j]);
    }
    const uint32_t picks = select_top_slots_small<kStepNT, kStepKPT, 1024>(key, (uint32_t)K, sm.T);
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kStepNT>((uint32_t)__popc(picks), sm.T.S.scan, &total);
#pragma unroll
    for (int j = 0; j < kStepKPT; ++j)
        if ((picks >> j) & 1u) atomicAdd(&sm.gpicked[(s0 + j) >> msh], 1u);
    lds_barrier();
    for (int g = tid; g < groups; g += kStepNT)
        if ((sm.gcount[g] & kGroupDropped) && sm.gpicked[g] == (uint32_t)m) sm.fail = 1;
    lds_barrier();
    if (sm.fail) {
        step_stream_exact(a.scores + (int64_t)t * a.stride, n, K, sm.T.S, sm.sel);
    } else {
#pragma unroll
        for (int j = 0; j < kStepKPT; ++j) {
            const bool pk = (picks >> j) & 1u;
            if (pk && pos < (uint32_t)kStepMaxK) sm.sel[pos] = id[j];
            pos += pk;
        }
    }
    lds_barrier();
    for (int i = tid; i < K; i += kStepNT) st_coh32(a.sel + (int64_t)t * K + i, (uint32_t)sm.sel[i]);
}

// ---------------------------------------------------------------- the kernel

__global__ __launch_bounds__(kStepNT, 1) void k_decode_step(StepArgs a) {
    __shared__ __attribute__((aligned(16))) StepSmem sm;
    __shared__ StepPlan plan;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    StepCounters* C = a.ctr;

    // ---- plan (identical in every workgroup)
    if (tid < 64) {
        int nv = 0, nt = 0;
        if (tid < a.T) {
            const int b = a.q_seq[tid];
            const int f = a.first_valid[b];
            const int qp = a.q_pos[tid];
            nv = qp >= f ? (qp - f + 1) >> 2 : 0;
            plan.nvis[tid] = nv;
            plan.first[tid] = f;
            plan.tail[tid] = qp >= f ? (qp - f + 1) - 4 * nv : 0;
            plan.pbase[tid] = a.pool_base[b];
            plan.rbase[tid] = a.row_base[b];
            nt = (nv + kSTile - 1) / kSTile;
            plan.ntiles[tid] = nt;
        }
        // rank by (tiles desc, index asc)
        int rank = 0;
        for (int u = 0; u < a.T; ++u) {
            const int nu = __shfl(nt, u, 64);
            rank += (nu > nt || (nu == nt && u < tid)) ? 1 : 0;
        }
        if (tid < a.T) plan.order[rank] = tid;
    }
    lds_barrier();
    const int hg = a.H / 16, per_t = a.splits * hg, per_c = a.splits > 1 ? a.H / kCombHeads : 0;
    if (tid == 0) {
        int x = 0, e = 0;
        auto add = [&](int stage, int r, int count) {
            if (count <= 0) return;
            plan.seg[e] = x;
            plan.seg_stage[e] = (uint8_t)stage;
            plan.seg_rank[e] = (uint8_t)r;
            ++e;
            x += count;
        };
        for (int r = 0; r <= a.T; ++r) {
            if (r < a.T) add(0, r, plan.ntiles[plan.order[r]]);
            if (r >= 1 && plan.nvis[plan.order[r - 1]] > a.select_k) add(1, r - 1, 1);
        }
        for (int r = 0; r < a.T; ++r) add(2, r, per_t);
        for (int r = 0; r < a.T; ++r) add(3, r, per_c);
        plan.seg[e] = x;
        plan.n_seg = e;
        plan.n_total = x;
    }
    lds_barrier();
    const int n_total = plan.n_total;

    // task -> (stage, query, index within the stage)
    auto locate = [&](int i, int& stage, int& t, int& j) {
        int lo = 0, hi = plan.n_seg - 1;                  // last segment with seg[e] <= i
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (plan.seg[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        stage = plan.seg_stage[lo];
        t = plan.order[plan.seg_rank[lo]];
        j = i - plan.seg[lo];
    };
    auto claim = [&]() -> uint32_t {
        return __hip_atomic_fetch_add(&C->queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // ---- scoring registers: the wave's two 64-pool groups of a task and the
    // task's query, loaded one task ahead (each group is reloaded as soon as
    // its MFMAs have consumed it).
    u32x4 v[2][16];
    IdxQuery Q;
    auto is_tile = [&](int i) {
        if (i >= n_total) return false;
        int st, t, j;
        locate(i, st, t, j);
        return st == 0;
    };
    // Pools p0 + 256 half + 64 wave .. +64 of query t (nothing when none is visible).
    auto load_half = [&](int t, int p0, int half) {
        const int g0 = uniform32(p0 + half * 256 + wave * 64);
        const int lim = plan.nvis[t] - g0;
        if (lim > 0) load_pool_group(a.pools + (plan.pbase[t] + g0) * kDI, lim, v[half]);
    };

    // ---- the task loop.  A run of consecutive scoring tasks is one inner loop
    // in which each task has its pools in registers (loaded one task ahead)
    // and has already claimed its successor; other tasks claim theirs when
    // done, so a long task never holds a claimed tile back.
    if (tid == 0) plan.task = (int)claim();
    lds_barrier();
    int cur = plan.task;
    lds_barrier();

    while (cur < n_total) {
        int stage, t, jj;
        locate(cur, stage, t, jj);
        if (stage == 0) {
          uint32_t pending = 0;
          {
            int st0, t0, j0;
            locate(cur, st0, t0, j0);
            load_half(t0, j0 * kSTile, 0);
            load_half(t0, j0 * kSTile, 1);
            load_idx_query(a.q_idx, a.w, t0, Q);
          }
          if (tid == 0) pending = claim();
          while (true) {
            locate(cur, stage, t, jj);
            if (tid == 0) plan.task = (int)pending;
            lds_barrier();
            const int nxt = plan.task;
            lds_barrier();
            const bool nxt_tile = is_tile(nxt);
            if (tid == 0 && nxt_tile) pending = claim();
            int nt = 0, np0 = 0;                               // the next task's query and first pool
            if (nxt_tile) {
                int st2, j2;
                locate(nxt, st2, nt, j2);
                np0 = j2 * kSTile;
            }
            // ============================ scoring tile
            const int p0 = jj * kSTile;
            const int nvis = plan.nvis[t];
            const int m = nvis > a.select_k ? group_quota<true>(a.select_k, nvis) : 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float s = score_pool_group(Q, v[half]);
                if (nxt_tile) {
                    load_half(nt, np0, half);
                    if (half == 1) load_idx_query(a.q_idx, a.w, nt, Q);
                }
                // lane l holds pool p0 + half*256 + wave*64 + l: lanes are in id order
                const int p = p0 + half * 256 + wave * 64 + lane;
                const bool valid = p < nvis;
                if (valid) st_coh32(a.scores + (int64_t)t * a.stride + p, __float_as_uint(s));
                if (m > 0)
                    keep_group_best(s, valid, p, (p0 + half * 256) / kSGroup + wave, m,
                                    a.cand + (int64_t)t * kStepCandCap, a.cand_n + (int64_t)t * kStepMaxGroups,
                                    [](uint64_t* q, uint64_t x) { st_coh64(q, x); },
                                    [](int32_t* q, uint32_t x) { st_coh32(q, x); });
            }
            if (nvis > a.select_k) publish(&C->tiles_done[t]);   // dense queries need no hand-off
            cur = nxt;
            if (!nxt_tile) break;
          }
          continue;
        }
        if (stage == 1) {
            // ============================ selection of one sparse query
            wait_counter(&C->tiles_done[t], (uint32_t)plan.ntiles[t], &C->error);
            step_select(a, sm.sel, plan, t);
            publish(&C->sel_ready[t]);
            lds_barrier();
        } else if (stage == 2) {
            // ============================ attention split
            const int split = jj / hg, head0 = 16 * (jj % hg);
            const int nvis = plan.nvis[t], K = min(a.select_k, nvis);
            const bool sparse = nvis > a.select_k;
            if (sparse) wait_counter(&C->sel_ready[t], 1u, &C->error);
            const int64_t rb = plan.rbase[t];
            const int f = plan.first[t], tail = plan.tail[t];
            const int32_t* selt = a.sel + (int64_t)t * a.select_k;
            auto idx_at = [&](int pos) -> int {
                if (pos < 4 * K) {
                    const int pool = sparse ? (int)ld_coh32(selt + (pos >> 2)) : (pos >> 2);
                    return (int)(rb + f + 4 * (int64_t)pool + (pos & 3));
                }
                if (pos < 4 * K + tail) return (int)(rb + f + 4 * (int64_t)nvis + (pos - 4 * K));
                return -1;
            };
            if (a.indices && head0 == 0)
                for (int pos = split * kRChunk + tid; pos < min(a.W, (split + 1) * kRChunk); pos += kStepNT)
                    a.indices[(int64_t)t * a.W + pos] = idx_at(pos);
            if (a.pool_ids && split == 0 && head0 == 0)
                for (int i = tid; i < a.select_k; i += kStepNT)
                    a.pool_ids[(int64_t)t * a.select_k + i] =
                        i < K ? (sparse ? (int)ld_coh32(selt + i) : i) : -1;
            mla_rows_split<2, true>(sm.mla, [&](int i) { return mla_q_piece<kStepNT>(a.q, t, a.H, head0, i); },
                                    a.cache, a.row_bytes, idx_at, a.W, a.H, a.scale_log2, t, head0, split, split,
                                    split + 1, a.splits, a.part_o, a.part_ml, a.out, a.out_f32, a.lse);
            if (a.splits > 1) publish(&C->splits_done[t]);
            lds_barrier();
        } else {
            // ============================ combine: 4 heads of one query
            const int h0 = jj * kCombHeads;
            wait_counter(&C->splits_done[t], (uint32_t)per_t, &C->error);
            const int S = a.splits;
            if (tid < 64 * kCombHeads && lane < 64) {
                const int hh = tid >> 6;
                MlaPartial pm = {-INFINITY, 0.f};
                if (lane < S) {
                    const uint64_t raw = ld_coh64(a.part_ml + ((int64_t)t * S + lane) * a.H + h0 + hh);
                    pm.m = __uint_as_float((uint32_t)raw);
                    pm.l = __uint_as_float((uint32_t)(raw >> 32));
                }
                const bool live = pm.l > 0.f;
                float Mx = live ? pm.m : -INFINITY;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, o, 64));
                const float wt = live ? exp2f(pm.m - Mx) : 0.f;
                float L = pm.l * wt;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
                if (lane < kMaxSplits) sm.comb.wgt[hh][lane] = wt;
                if (lane == 0) {
                    sm.comb.M[hh] = Mx;
                    sm.comb.L[hh] = L;
                }
            }
            lds_barrier();
            {
                const int hh = tid >> 6, c0 = (tid & 63) * 8;
                const int head = h0 + hh;
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
                // the query's partials: one wave-uniform descriptor, per-lane offsets
                const float* pq = a.part_o + (int64_t)t * S * a.H * kD;
                const __amdgpu_buffer_rsrc_t rs = coh_rsrc(pq, (uint32_t)(S * a.H * kD * 4));
                for (int s = 0; s < S; ++s) {
                    const float wt = sm.comb.wgt[hh][s];
                    if (wt > 0.f) {
                        const uint32_t off = (uint32_t)(((s * a.H + head) * kD + c0) * 4);
                        const u32x4 r0 = ld_coh128(rs, off), r1 = ld_coh128(rs, off + 16);
                        acc0 += __builtin_bit_cast(f32x4, r0) * wt;
                        acc1 += __builtin_bit_cast(f32x4, r1) * wt;
                    }
                }
                const float L = sm.comb.L[hh];
                const float inv = L > 0.f ? 1.0f / L : 0.f;
                acc0 *= inv;
                acc1 *= inv;
                const int64_t orow = ((int64_t)t * a.H + head) * kD + c0;
                if (a.out_f32) {
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow) = acc0;
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow + 4) = acc1;
                } else {
                    u32x4 pk;
                    pk[0] = f32_to_bf16_rne(acc0[0]) | (f32_to_bf16_rne(acc0[1]) << 16);
                    pk[1] = f32_to_bf16_rne(acc0[2]) | (f32_to_bf16_rne(acc0[3]) << 16);
                    pk[2] = f32_to_bf16_rne(acc1[0]) | (f32_to_bf16_rne(acc1[1]) << 16);
                    pk[3] = f32_to_bf16_rne(acc1[2]) | (f32_to_bf16_rne(acc1[3]) << 16);
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + orow) = pk;
                }
                if (a.lse && (tid & 63) == 0)
                    a.lse[(int64_t)t * a.H + head] = L > 0.f ? (sm.comb.M[hh] + log2f(L)) * kLn2 : -INFINITY;
            }
            lds_barrier();
        }
        if (tid == 0) plan.task = (int)claim();
        lds_barrier();
        cur = plan.task;
        lds_barrier();
    }
    // ---- past the last task: the last workgroup out resets the queue
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&C->exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == (uint32_t)a.grid) {
            for (int q = 0; q < a.T; ++q) {
                st_coh32(&C->tiles_done[q], 0u);
                st_coh32(&C->sel_ready[q], 0u);
                st_coh32(&C->splits_done[q], 0u);
            }
            st_coh32(&C->queue, 0u);
            st_coh32(&C->exited, 0u);
        }
    }
}

}  // namespace dsa

namespace dsa_host {

static size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StepLayout {
    size_t ctr, scores, cand, cand_n, sel, part_o, part_ml, total;
};

static StepLayout step_layout(const dsa_dims& d, int32_t T, int32_t stride, int splits) {
    StepLayout L{};
    size_t o = 0;
    L.ctr = o;
    o += r256(sizeof(dsa::StepCounters));
    L.scores = o;
    o += r256((size_t)T * stride * 4);
    L.cand = o;
    o += r256((size_t)T * dsa::kStepCandCap * 8);
    L.cand_n = o;
    o += r256((size_t)T * dsa::kStepMaxGroups * 4);
    L.sel = o;
    o += r256((size_t)T * (d.index_topk / d.kpool) * 4);
    L.part_o = o;
    o += r256(splits > 1 ? (size_t)T * splits * d.mla_heads * dsa::kD * 4 : 0);
    L.part_ml = o;
    o += r256(splits > 1 ? (size_t)T * splits * d.mla_heads * sizeof(dsa::MlaPartial) : 0);
    L.total = o;
    return L;
}

static int step_splits(const dsa_dims& d) { return (int)cdiv(d.out_width, dsa::kRChunk); }

bool decode_step_supported(const dsa_dims& d, int32_t T, int32_t stride) {
    const int sk = d.index_topk / d.kpool;
    return d.idx_heads == 32 && d.idx_dim == 128 && d.kpool == 4 && d.latent_dim == dsa::kD &&
           d.mla_heads % 16 == 0 && d.mla_heads <= 64 && sk <= dsa::kStepMaxK && T <= dsa::kStepMaxT &&
           stride <= dsa::kStepMaxGroups * dsa::kSGroup && step_splits(d) <= dsa::kMaxSplits;
}

size_t decode_step_workspace_bytes(const dsa_dims& d, int32_t T, int32_t stride) {
    if (T <= 0) return 0;
    return step_layout(d, T, stride, step_splits(d)).total;
}

hipError_t launch_decode_step(const dsa_dims& d, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                              const dsa_seqs& seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                              int32_t stride, const uint16_t* q, const int8_t* cache, float scale, void* out,
                              int out_dtype, float* lse, int32_t* pool_ids, int32_t* indices, void* ws,
                              hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int splits = step_splits(d);
    const StepLayout L = step_layout(d, T, stride, splits);
    char* base = reinterpret_cast<char*>(ws);
    dsa::StepArgs a{};
    a.T = T;
    a.H = d.mla_heads;
    a.W = d.out_width;
    a.select_k = d.index_topk / d.kpool;
    a.stride = stride;
    a.splits = splits;
    a.grid = device_info().cu_count;
    a.scale_log2 = scale * dsa::kLog2e;
    a.q_idx = q_idx;
    a.w = w;
    a.pools = pools;
    a.first_valid = seqs.first_valid;
    a.pool_base = seqs.pool_base;
    a.row_base = seqs.row_base;
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.q = q;
    a.cache = reinterpret_cast<const uint8_t*>(cache);
    a.row_bytes = d.row_bytes;
    a.out = out;
    a.out_f32 = out_dtype == DSA_F32;
    a.lse = lse;
    a.pool_ids = pool_ids;
    a.indices = indices;
    a.ctr = reinterpret_cast<dsa::StepCounters*>(base + L.ctr);
    a.scores = reinterpret_cast<float*>(base + L.scores);
    a.cand = reinterpret_cast<uint64_t*>(base + L.cand);
    a.cand_n = reinterpret_cast<int32_t*>(base + L.cand_n);
    a.sel = reinterpret_cast<int32_t*>(base + L.sel);
    a.part_o = reinterpret_cast<float*>(base + L.part_o);
    a.part_ml = reinterpret_cast<dsa::MlaPartial*>(base + L.part_ml);
    hipLaunchKernelGGL(dsa::k_decode_step, dim3((unsigned)a.grid), dim3(dsa::kStepNT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa_host
