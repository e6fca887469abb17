// Per-wave scoring of one 64-pool group for the 32-head x 128 indexer
// ([Ref] Functions: index_scores -- score[p] = sum_h w[h] * relu(q[h] . pool[p])).
//
// The contraction q (32 heads x 128) x pool^T (128 x 64 pools) runs on
// v_mfma_f32_16x16x32_bf16 with the B operand loaded straight from HBM into
// registers: no LDS staging, no barrier, so a wave starts its MFMAs as soon as
// its own 16 KB has arrived.  With lane l = 16 * g + c:
//   B (N-tile r, K-step s): pool 16 r + c, dims 32 s + 8 g .. +8  -- each load
//     instruction reads 64 contiguous bytes of 16 pool rows;
//   A (M-tile mt, K-step s): head 16 mt + c, the same dims;
//   D (N-tile r, M-tile mt): pool 16 r + c, heads 16 mt + 4 g + i.
// The ReLU and head weighting run on the accumulators; a two-stage
// reduce-scatter over the lane groups g (xor 32, then xor 16) leaves the score
// of pool l in lane l, so lanes are in pool order for the group selection.
// Every kernel that scores decode pools uses these three functions, so the
// separate and the single-launch decode paths agree bit for bit.
#pragma once
#include "dsa_common.h"

namespace dsa {

constexpr int kHI = 32, kDI = 128;

struct IdxQuery {
    u32x4 a[2][4];   // [M-tile][K-step]
    f32x4 w[2];      // heads 16 mt + 4 g + i
};

// Loads go through raw buffer descriptors over wave-uniform bases; a lane
// offset is one VGPR (row c of a 16-row block, 16-byte chunk g) and the
// constant part of each address rides in the SGPR offset.  Every access is
// kept inside the buffer by the offsets themselves: the descriptor's range
// check does not cover the SGPR offset.

// Query t's A operand and head weights (t wave-uniform).
__device__ __forceinline__ void load_idx_query(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                                               int64_t t, IdxQuery& Q) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q_idx + t * (kHI * kDI), kHI * kDI * 2);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(w + t * kHI, kHI * 4);
    const uint32_t loff = (uint32_t)(c * (kDI * 2) + 16 * g);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) Q.a[mt][s] = ld_buf128(rq, loff, (uint32_t)(16 * mt * (kDI * 2) + 64 * s));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        Q.w[mt] = __builtin_bit_cast(f32x4, ld_buf128(rw, (uint32_t)(16 * g), (uint32_t)(64 * mt)));
}

// The same operand from a copy of q in LDS ([head][dim], row stride qs
// elements) and the head weights in LDS.
__device__ __forceinline__ void load_idx_query_lds(const uint16_t* q_lds, int qs, const float* w_lds, IdxQuery& Q) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            Q.a[mt][s] = *reinterpret_cast<const u32x4*>(&q_lds[(16 * mt + c) * qs + 32 * s + 8 * g]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) Q.w[mt] = *reinterpret_cast<const f32x4*>(&w_lds[16 * mt + 4 * g]);
}

// rows: the group's first pool row (wave-uniform); lim (>= 1): rows of the
// group that exist.  Rows at or past lim re-read row lim - 1, so every access
// stays inside the group's existing rows (their scores are meaningless and
// the caller masks them).
__device__ __forceinline__ void load_pool_group(const uint16_t* __restrict__ rows, int lim, u32x4 (&v)[16]) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rows, (uint32_t)(min(lim, 64) * (kDI * 2)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t loff = (uint32_t)(min(16 * r + c, lim - 1) * (kDI * 2) + 16 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) v[4 * r + s] = ld_buf128(rr, loff, (uint32_t)(64 * s));
    }
}

// Returns the score of pool (lane) of the group.
__device__ __forceinline__ float score_pool_group(const IdxQuery& Q, const u32x4 (&v)[16]) {
    const int lane = threadIdx.x & 63;
    float part[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc0 = mfma16(as_bf16x8(Q.a[0][s]), as_bf16x8(v[4 * r + s]), acc0);
            acc1 = mfma16(as_bf16x8(Q.a[1][s]), as_bf16x8(v[4 * r + s]), acc1);
        }
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += Q.w[0][i] * fmaxf(acc0[i], 0.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += Q.w[1][i] * fmaxf(acc1[i], 0.f);
        part[r] = sum;
    }
    // Lane group g holds a partial of pools 16 r + c for every r; lane group
    // g ends with the full sum of N-tile r = g.
    const bool h = (lane & 32) != 0;     // keeps N-tiles 2h, 2h + 1
    const float k0 = (h ? part[2] : part[0]) + __shfl_xor(h ? part[0] : part[2], 32, 64);
    const float k1 = (h ? part[3] : part[1]) + __shfl_xor(h ? part[1] : part[3], 32, 64);
    const bool j = (lane & 16) != 0;     // keeps N-tile 2h + j
    return (j ? k1 : k0) + __shfl_xor(j ? k0 : k1, 16, 64);
}

// The score of one more pool, given as a single N-tile's B operand b[s]
// (column c = lane % 16 holds it in every lane group): lane l gets exactly
// what score_pool_group returns in lane l for a group whose N-tile l / 16
// column l % 16 holds that pool -- the same MFMAs, the same per-lane partial
// and the same two shuffle-adds in the same order.
__device__ __forceinline__ float score_pool_column(const IdxQuery& Q, const u32x4 (&b)[4]) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        acc0 = mfma16(as_bf16x8(Q.a[0][s]), as_bf16x8(b[s]), acc0);
        acc1 = mfma16(as_bf16x8(Q.a[1][s]), as_bf16x8(b[s]), acc1);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += Q.w[0][i] * fmaxf(acc0[i], 0.f);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += Q.w[1][i] * fmaxf(acc1[i], 0.f);
    const float k = sum + __shfl_xor(sum, 32, 64);
    return k + __shfl_xor(k, 16, 64);
}

}  // namespace dsa
