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

// part[r]: this lane's partial of pool 16 r + c.  Lane group g holds a
// partial of pools 16 r + c for every r; lane group g ends with the full sum
// of N-tile r = g, so lane l holds pool l.
__device__ __forceinline__ float reduce_group_parts(const float (&part)[4]) {
    // lane half h keeps N-tiles 2h, 2h + 1, then row j of it N-tile 2h + j
    const float k0 = add_swap32(part[0], part[2]);
    const float k1 = add_swap32(part[1], part[3]);
    return add_swap16(k0, k1);
}

// Returns the score of pool (lane) of the group.
__device__ __forceinline__ float score_pool_group(const IdxQuery& Q, const u32x4 (&v)[16]) {
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
        for (int i = 0; i < 4; ++i) sum += Q.w[0][i] * relu_bits(acc0[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += Q.w[1][i] * relu_bits(acc1[i]);
        part[r] = sum;
    }
    return reduce_group_parts(part);
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
    for (int i = 0; i < 4; ++i) sum += Q.w[0][i] * relu_bits(acc0[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += Q.w[1][i] * relu_bits(acc1[i]);
    const float k = add_swap32(sum, sum);
    return add_swap16(k, k);
}

// ------------------------------------------------------------------ INT8 pools
// Pools stored as INT8 codes (128-byte rows) with one fp32 scale per pool
// ([Flash] What is quantized: the INT8 indexer cache).  For pool p with scale
// s_p > 0, relu(q . (s_p code_p)) = s_p relu(q . code_p), so
//   score[p] = s_p * sum_h w[h] * relu(q[h] . code_p),
// one multiply per pool after the head sum.  The codes go into the B operand
// as bf16 of (code + 128) (exact; one conversion per code), and the bias is
// taken off the dot products exactly as the bf16 sum 128 * sum_d q[h][d]
// (computed once per tile in fp32).
// Lane l = 16 g + c loads, for N-tile r, bytes 32 g .. 32 g + 32 of pool
// 16 r + c (two 16-byte loads: dims 32 g .. 32 g + 31); K-step s uses dims
// 32 g + 8 s .. + 8 of them.  The reduction axis is permuted the same way in
// the A operand (load_idx_query_lds_i8), so the products are unchanged.

struct IdxQueryI8 {
    IdxQuery q;        // A operand in the permuted order, head weights
    f32x4 bias[2];     // 128 * sum_d q[h][d] for heads 16 mt + 4 g + i
};

__device__ __forceinline__ void load_idx_query_lds_i8(const uint16_t* q_lds, int qs, const float* w_lds,
                                                      IdxQueryI8& Q) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    float qsum[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            Q.q.a[mt][s] = *reinterpret_cast<const u32x4*>(&q_lds[(16 * mt + c) * qs + 32 * g + 8 * s]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc += bf16_to_f32(Q.q.a[mt][s][e] & 0xFFFFu) + bf16_to_f32(Q.q.a[mt][s][e] >> 16);
        }
        acc = add_swap16(acc, acc);
        qsum[mt] = add_swap32(acc, acc);                   // head 16 mt + c, in every lane group
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        Q.q.w[mt] = *reinterpret_cast<const f32x4*>(&w_lds[16 * mt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) Q.bias[mt][i] = 128.0f * __shfl(qsum[mt], 4 * g + i, 64);
    }
}

// rows: the group's first code row (wave-uniform); lim (>= 1) rows exist;
// rows at or past lim re-read row lim - 1 (masked by the caller).
__device__ __forceinline__ void load_pool_group_i8(const int8_t* __restrict__ rows, int lim, u32x4 (&v)[8]) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rows, (uint32_t)(min(lim, 64) * kDI));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t loff = (uint32_t)(min(16 * r + c, lim - 1) * kDI + 32 * g);
#pragma unroll
        for (int j = 0; j < 2; ++j) v[2 * r + j] = ld_buf128(rr, loff, (uint32_t)(16 * j));
    }
}

// K-step s of the B operand from this lane's 32 code bytes (w0 = bytes 0-15, w1 = bytes 16-31).
__device__ __forceinline__ u32x4 i8_kstep(const u32x4& w0, const u32x4& w1, int s) {
    const u32x4& w = s < 2 ? w0 : w1;
    return codes8_to_biased_bf16(w[(s & 1) * 2], w[(s & 1) * 2 + 1]);
}

// The head sum of one N-tile's accumulators (heads 16 mt + 4 g + i), bias off.
__device__ __forceinline__ float i8_head_sum(const IdxQueryI8& Q, const f32x4& acc0, const f32x4& acc1) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += Q.q.w[0][i] * relu_bits(acc0[i] - Q.bias[0][i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += Q.q.w[1][i] * relu_bits(acc1[i] - Q.bias[1][i]);
    return sum;
}

// Score of pool (lane) of the group; scale: that pool's scale.
__device__ __forceinline__ float score_pool_group_i8(const IdxQueryI8& Q, const u32x4 (&v)[8], float scale) {
    float part[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 b = i8_kstep(v[2 * r], v[2 * r + 1], s);
            acc0 = mfma16(as_bf16x8(Q.q.a[0][s]), as_bf16x8(b), acc0);
            acc1 = mfma16(as_bf16x8(Q.q.a[1][s]), as_bf16x8(b), acc1);
        }
        part[r] = i8_head_sum(Q, acc0, acc1);
    }
    return reduce_group_parts(part) * scale;
}

// One more pool as a single N-tile column (its 32 code bytes for this lane
// group in w0, w1 in every lane of the group): lane l gets exactly what
// score_pool_group_i8 returns in lane l for a group holding that pool there.
__device__ __forceinline__ float score_pool_column_i8(const IdxQueryI8& Q, const u32x4& w0, const u32x4& w1,
                                                      float scale) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const u32x4 b = i8_kstep(w0, w1, s);
        acc0 = mfma16(as_bf16x8(Q.q.a[0][s]), as_bf16x8(b), acc0);
        acc1 = mfma16(as_bf16x8(Q.q.a[1][s]), as_bf16x8(b), acc1);
    }
    const float sum = i8_head_sum(Q, acc0, acc1);
    const float k = add_swap32(sum, sum);
    return add_swap16(k, k) * scale;
}

}  // namespace dsa
