// Device code shared by the sparse MLA kernels: the 16-head row-split
// attention (k_mla_rows and the fused decode step) and its building blocks.
// The design notes are at the top of sparse_mla.hip.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kD = 512;
constexpr int kChunk = 64;
constexpr int kKVRow = kD + 8;       // bf16 elements per LDS row (1040 B)
constexpr int kPRow = kChunk + 8;    // bf16 elements per P' row (144 B)
constexpr int kMaxSplitRows = 2176;  // index entries one split may cover (staged in LDS)
constexpr int kMaxSplits = 64;       // list partitions per query
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct alignas(8) MlaPartial {
    float m;   // running max, log2 domain
    float l;   // running sum
};

// 4 INT8 codes -> 4 bf16 of the signed codes.  Each code is sign-extended
// from its byte inside the conversion (hipcc selects v_cvt_f32_i32 with an
// SDWA sext byte operand: one instruction a code, no extract or bias).
__device__ __forceinline__ void int8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const float f0 = (float)(int32_t)(int8_t)(w & 0xFFu);
    const float f1 = (float)(int32_t)(int8_t)((w >> 8) & 0xFFu);
    const float f2 = (float)(int32_t)(int8_t)((w >> 16) & 0xFFu);
    const float f3 = (float)((int32_t)w >> 24);
    // Small integers are exact in bf16: keep the upper halves.
    lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// ------------------------------------------------------------------ k_mla_rows
constexpr int kRChunk = 128;          // list positions per chunk of k_mla_rows and the fused step
constexpr int kRStride = kD + 8;      // bf16 elements per LDS row
constexpr float kLazyMax = 8.0f;      // raise the running max only beyond 2^8

// Physical row (within a 16-row tile) of MFMA row slot s: bits 2 and 3 swapped.
__device__ __forceinline__ int row_of_slot(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }


// LDS of one split walking chunks of 16 * RT * NW rows (NW waves of RT
// 16-row tiles).
template <int RT, int NW = 4>
struct MlaRowsSmemT {
    static constexpr int kRows = 16 * RT * NW;
    static constexpr int kPLS = kRows + 8;   // bf16 per head row of P'
    uint16_t kv[kRows * kRStride];           // the chunk's rows as bf16 (code + 128)
    uint16_t qs[16 * kRStride];              // the 16 heads of q, [head][dim]
    uint16_t pl[2][16 * kPLS];               // P' hi, lo: [head][row]
    float red_max[NW][16];
    float red_l[NW][16];
    float red_p[NW][16];
};
using MlaRowsSmem = MlaRowsSmemT<2>;         // 128-row chunks (kRChunk)


// Output stores of a split: plain, or agent-coherent (relaxed agent-scope
// atomic stores, which bypass the non-coherent L2 so that a workgroup on
// another XCD of the same launch reads what was written).
template <bool COH>
__device__ __forceinline__ void store_f32x4(float* p, f32x4 v) {
    if constexpr (COH) {
        uint64_t* q = reinterpret_cast<uint64_t*>(p);
        __hip_atomic_store(q, ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *reinterpret_cast<f32x4*>(p) = v;
    }
}

template <bool COH>
__device__ __forceinline__ void store_partial(MlaPartial* p, MlaPartial v) {
    if constexpr (COH) {
        __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                           ((uint64_t)__float_as_uint(v.l) << 32) | __float_as_uint(v.m), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *p = v;
    }
}

// This thread's pieces of q (see mla_q_piece) into the padded LDS rows the
// waves read it from.
template <int NT, int QP>
__device__ __forceinline__ void mla_stage_q(uint16_t* qs, const u32x4 (&qv)[QP]) {
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int k = threadIdx.x + NT * i;            // 16-byte piece k: head k / 64, dims 8 (k % 64) ..
        *reinterpret_cast<u32x4*>(&qs[(k >> 6) * kRStride + 8 * (k & 63)]) = qv[i];
    }
}

// 16-byte piece i of this thread's share of q (16 heads x 512 bf16 of query
// t from head0; piece k = tid + NT i holds head k / 64, dims 8 (k % 64) ..).
template <int NT>
__device__ __forceinline__ u32x4 mla_q_piece(const uint16_t* __restrict__ q, int t, int H, int head0, int i) {
    return *reinterpret_cast<const u32x4*>(q + ((int64_t)t * H + head0) * kD + 8 * (threadIdx.x + NT * i));
}

// One split of k_mla_rows: query t, heads [head0, head0 + 16), list chunks
// [c_begin, c_end) of 16 * RT * NW positions (each of the NW waves owns RT
// 16-row tiles of a chunk and 512 / NW columns of the output).  idx_at(pos)
// gives the cache row of list position pos (< W), or a negative value for an
// empty slot; q_piece(i) gives piece i of this thread's share of q (see
// mla_q_piece), loaded there or earlier.  COH makes the partial results
// agent-coherent (read back by another workgroup of the same launch) instead
// of plain stores.  Every thread of the block must call it; it contains
// workgroup barriers.
template <int RT, bool COH, int NW = 4, bool QS_READY = false, class IdxFn, class QFn>
__device__ __forceinline__ void mla_rows_split(
    MlaRowsSmemT<RT, NW>& sm, QFn q_piece, const uint8_t* __restrict__ cache, int row_bytes,
    IdxFn idx_at, int W, int H, float scale_log2, int t, int head0, int split, int c_begin, int c_end,
    int splits, float* __restrict__ part_o, MlaPartial* __restrict__ part_ml, void* __restrict__ out,
    int out_f32, float* __restrict__ lse) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    const int prow = row_of_slot(n16);            // row (within a 16-row tile) this lane loads
    const int srow = row_of_slot(4 * g4);         // first of the 4 rows this lane's S^T values cover
    constexpr int NT = 64 * NW;
    constexpr int CH = 16 * RT * NW;              // rows per chunk
    constexpr int PLS = MlaRowsSmemT<RT, NW>::kPLS;
    constexpr int NKS = CH / 32;                  // 32-row k-steps of O^T += V^T P'^T
    constexpr int CW = kD / NW;                   // output columns per wave
    constexpr int NG = CW / 64;                   // 64-column groups per wave
    constexpr int QP = 16 * kD * 2 / 16 / NT;     // 16-byte pieces of q per thread
    static_assert(NG >= 1 && QP >= 1 && CH % 32 == 0, "unsupported split shape");

    auto load_idx = [&](int c, int* id) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int pos = c * CH + 16 * RT * w + 16 * rt + prow;
            id[rt] = pos < W ? idx_at(pos) : -1;
        }
    };
    u32x4 raw[RT][8];
    float rsc[RT];
    auto load_rows = [&](const int* id) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (id[rt] >= 0) {
                const uint8_t* src = cache + (int64_t)id[rt] * row_bytes;
#pragma unroll
                for (int i = 0; i < 8; ++i) raw[rt][i] = *reinterpret_cast<const u32x4*>(src + 64 * i + 16 * g4);
                rsc[rt] = *reinterpret_cast<const float*>(src + kD);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) raw[rt][i] = u32x4{0u, 0u, 0u, 0u};
                rsc[rt] = -1.0f;                 // marks an empty slot
            }
        }
    };

    // The index loads go out first (the rows wait on them, and loads complete
    // in issue order as far as the wait counters go), then q (16 heads x 512,
    // 16 KB, read once per workgroup, 64 bytes per thread, handed to the
    // waves through LDS), then the first chunk's rows.
    int id_cur[RT], id_next[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) id_cur[rt] = id_next[rt] = -1;
    if (c_begin < c_end) {
        load_idx(c_begin, id_cur);
        if (c_begin + 1 < c_end) load_idx(c_begin + 1, id_next);
    }
    if constexpr (QS_READY) {
        // the caller has staged q in sm.qs (mla_stage_q) behind a barrier
        if (c_begin < c_end) load_rows(id_cur);
    } else {
        u32x4 qv[QP];
#pragma unroll
        for (int i = 0; i < QP; ++i) qv[i] = q_piece(i);
        if (c_begin < c_end) load_rows(id_cur);
        mla_stage_q<NT>(sm.qs, qv);
        lds_barrier();
    }

    // Q^T operand (B of S^T): head head0 + n16, reduction index
    // 64 (j/2) + 16 g4 + 8 (j%2) + e -- the bytes this lane holds of its row.
    // (The padded head rows make these 16-byte LDS reads conflict free.)
    u32x4 qb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        qb[j] = *reinterpret_cast<const u32x4*>(&sm.qs[n16 * kRStride + 64 * (j >> 1) + 16 * g4 + 8 * (j & 1)]);
    // The K and V operands hold code + 128 (exact in bf16, one conversion per
    // code); the bias is removed afterwards: S -= 128 * sum_k q_k per head and
    // O -= 128 * sum_j P'_j over the same bf16 P' values the products used.
    float qsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qsum += bf16_to_f32(qb[j][k] & 0xFFFFu) + bf16_to_f32(qb[j][k] >> 16);
    qsum = add_swap16(qsum, qsum);
    qsum = add_swap32(qsum, qsum);
    const float sbias = 128.0f * qsum;

    // Running softmax state of head n16 (the same in every wave); l and the
    // P' sum cover this lane's own rows and are added up at the end.
    float m_run = -INFINITY, l_run = 0.f, p_run = 0.f;
    f32x4 acc[NG][4];                            // O^T: cols CW w + 64G + 16g4 + 4i + u, head n16
#pragma unroll
    for (int G = 0; G < NG; ++G)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[G][u] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = c_begin; c < c_end; ++c) {
        // A wave with no row in the chunk skips its work.  With one tile per
        // wave, a 32-row k-step of the PV product spans two waves, so every
        // wave stages its rows (empty ones hold code 0 with P' = 0).
        bool any = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) any = any || id_cur[rt] >= 0;
        const bool live = RT == 1 || __ballot(any) != 0ull;
        float rs_now[RT];
        f32x4 s[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            rs_now[rt] = rsc[rt];
            s[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (live) {
            // ---- convert this wave's rows, S^T = K Q^T (2 RT independent
            //      accumulation chains), and stage the rows for V^T
            f32x4 sc4[RT][2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sc4[rt][0] = sc4[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const u32x4 kb =
                        codes8_to_biased_bf16(raw[rt][j >> 1][(j & 1) * 2], raw[rt][j >> 1][(j & 1) * 2 + 1]);
                    sc4[rt][j & 1] = mfma16(as_bf16x8(kb), as_bf16x8(qb[j]), sc4[rt][j & 1]);
                    *reinterpret_cast<u32x4*>(
                        &sm.kv[(16 * RT * w + 16 * rt + prow) * kRStride + 64 * (j >> 1) + 16 * g4 + 8 * (j & 1)]) = kb;
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) s[rt] = sc4[rt][0] + sc4[rt][1];
        }
        // ---- next chunk's rows in flight while this one computes
        if (c + 1 < c_end) {
            load_rows(id_next);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) id_cur[rt] = id_next[rt];
            if (c + 2 < c_end) load_idx(c + 2, id_next);
        }

        // ---- chunk max per head across the NW waves (lane: head n16, rows slot 4*g4 + i)
        float z[RT][4], sc[RT][4];
        float cmax = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[rt][i] = __shfl(rs_now[rt], 4 * g4 + i, 64);
                z[rt][i] = sc[rt][i] > 0.f ? (s[rt][i] - sbias) * (sc[rt][i] * scale_log2) : -INFINITY;
                cmax = fmaxf(cmax, z[rt][i]);
            }
        cmax = max_swap16(cmax, cmax);
        cmax = max_swap32(cmax, cmax);
        if (g4 == 0) sm.red_max[w][n16] = cmax;
        lds_barrier();
        float wmax[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) wmax[k] = sm.red_max[k][n16];
        float chunk_max = wmax[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) chunk_max = fmaxf(chunk_max, wmax[k]);
        // k-steps with a live row (their source waves' maxima): the same
        // answer for every head.
        bool src_live[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            bool lv = false;
#pragma unroll
            for (int k = 0; k < NW; ++k)                // wave k's rows start at 16 RT k
                if ((16 * RT * k) / 32 == ks) lv = lv || wmax[k] != -INFINITY;
            src_live[ks] = __ballot(lv) != 0ull;
        }

        // The running max is raised only when the chunk exceeds it by 2^8.
        const float m_new = (m_run == -INFINITY || chunk_max > m_run + kLazyMax) ? chunk_max : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        if (__ballot(alpha != 1.0f && m_run != -INFINITY) != 0ull) {
#pragma unroll
            for (int G = 0; G < NG; ++G)
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[G][u] *= alpha;
        }
        l_run *= alpha;
        p_run *= alpha;
        m_run = m_new;

        // ---- P' = p * scale as bf16 hi + lo, to LDS as [head][row]
        uint32_t bh[RT][2], bl[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                float x[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i = 2 * i2 + h;
                    const float p = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[rt][i] - m_new);
                    l_run += p;
                    x[h] = p * fmaxf(sc[rt][i], 0.f);
                }
                uint32_t hp, lp;
                split_bf16x2(x[0], x[1], hp, lp);
                bh[rt][i2] = hp;
                bl[rt][i2] = lp;
                p_run += (__uint_as_float(hp << 16) + __uint_as_float(lp << 16)) +
                         (__uint_as_float(hp & 0xFFFF0000u) + __uint_as_float(lp & 0xFFFF0000u));
            }
        if (live) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int r0 = 16 * RT * w + 16 * rt + srow;
                *reinterpret_cast<u32x2*>(&sm.pl[0][n16 * PLS + r0]) = u32x2{bh[rt][0], bh[rt][1]};
                *reinterpret_cast<u32x2*>(&sm.pl[1][n16 * PLS + r0]) = u32x2{bl[rt][0], bl[rt][1]};
            }
        }
        lds_barrier();                               // rows and P' of all waves visible

        // ---- O^T += V^T P'^T over the chunk's rows, this wave's CW columns
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (!src_live[ks]) continue;             // no staged row in these 32
            const int r0 = 32 * ks + 8 * g4;         // k-slot e <-> row r0 + e
            const bf16x8 p_hi = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.pl[0][n16 * PLS + r0]));
            const bf16x8 p_lo = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.pl[1][n16 * PLS + r0]));
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                const uint16_t* vb = &sm.kv[r0 * kRStride + CW * w + 64 * G + 4 * n16];
                u32x2 v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const u32x2*>(vb + e * kRStride);
                u32x4 a[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int wd = u >> 1;
                    const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
                    a[u][0] = __builtin_amdgcn_perm(v[1][wd], v[0][wd], sel);
                    a[u][1] = __builtin_amdgcn_perm(v[3][wd], v[2][wd], sel);
                    a[u][2] = __builtin_amdgcn_perm(v[5][wd], v[4][wd], sel);
                    a[u][3] = __builtin_amdgcn_perm(v[7][wd], v[6][wd], sel);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[G][u] = mfma16(as_bf16x8(a[u]), p_hi, acc[G][u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[G][u] = mfma16(as_bf16x8(a[u]), p_lo, acc[G][u]);
            }
        }
        if (c + 1 < c_end) lds_barrier();            // rows and P' are rewritten next
    }

    // ---- totals over the NW waves' rows, then this wave's CW columns out
    // rows 0 and 2 carry l, rows 1 and 3 p: after the two swaps lanes 0..15
    // hold the wave's l totals and lanes 16..31 its p totals (the sums of the
    // xor-16, then xor-32 butterfly, bit for bit)
    const float lp = add_swap32(add_swap16(l_run, p_run), add_swap16(l_run, p_run));
    if (g4 == 0) sm.red_l[w][n16] = lp;
    if (g4 == 1) sm.red_p[w][n16] = lp;
    lds_barrier();
    float L = 0.f, PS = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        L += sm.red_l[k][n16];
        PS += sm.red_p[k][n16];
    }
    const float obias = 128.0f * PS;
    const int head = head0 + n16;
    if (splits == 1) {
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const int64_t orow = ((int64_t)t * H + head) * kD;
#pragma unroll
        for (int G = 0; G < NG; ++G)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = CW * w + 64 * G + 16 * g4 + 4 * i;
                const f32x4 o = (f32x4{acc[G][0][i], acc[G][1][i], acc[G][2][i], acc[G][3][i]} - obias) * inv;
                if (out_f32) {
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow + col) = o;
                } else {
                    u32x2 pk;
                    pk[0] = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
                    pk[1] = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
                    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + orow + col) = pk;
                }
            }
        if (lse && w == 0 && g4 == 0) lse[(int64_t)t * H + head] = L > 0.f ? (m_run + log2f(L)) * kLn2 : -INFINITY;
    } else {
        const int64_t slot = ((int64_t)t * splits + split) * H + head;
        if (L > 0.f) {
            float* po = part_o + slot * kD;
#pragma unroll
            for (int G = 0; G < NG; ++G)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = CW * w + 64 * G + 16 * g4 + 4 * i;
                    store_f32x4<COH>(po + col, f32x4{acc[G][0][i], acc[G][1][i], acc[G][2][i], acc[G][3][i]} - obias);
                }
        }
        if (w == 0 && g4 == 0) store_partial<COH>(part_ml + slot, MlaPartial{m_run, L});
    }
}

}  // namespace dsa
