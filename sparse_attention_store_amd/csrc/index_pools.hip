// index_pools: kpool-token pools of LayerNorm'd indexer keys, weighted by a
// per-channel softmax over the pool slots ([Ref] Traps: LayerNorm with bias,
// softmax over the slot axis, pools from the first valid token, full pools
// only; Functions: pool_states, layer_norm).
//
// One wave per pool.  A lane owns idx_dim/64 channels (2 for 128), reads the
// kpool token rows of k and gate (4 x 256 B each per pool, coalesced), takes
// mean and biased variance of each token row with two wave sums, and does the
// slot softmax in registers: no cross-lane step is needed for it because the
// softmax runs along the slot axis of a fixed channel.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

template <typename T>
__device__ __forceinline__ float load_val(const T* p);
template <> __device__ __forceinline__ float load_val<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_val<float>(const float* p) { return *p; }

template <int DI, typename T>
__global__ __launch_bounds__(256) void k_index_pools(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end,
    uint16_t* __restrict__ pools) {
    constexpr int KP = 4;
    constexpr int CPL = DI >= 64 ? DI / 64 : 1;       // channels per lane
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.y;
    const int p = pool_begin[b] + blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= pool_end[b]) return;
    const bool active = DI >= 64 || lane < DI;
    const int c0 = active ? lane * CPL : 0;
    const int64_t tok0 = tok_base[b] + first_valid[b] + (int64_t)KP * p;

    float wv[CPL], bv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { wv[c] = ln_w[c0 + c]; bv[c] = ln_b[c0 + c]; }

    float y[KP][CPL], g[KP][CPL];
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        const T* kr = k + (tok0 + s) * DI + c0;
        const T* gr = gate + (tok0 + s) * DI + c0;
        float x[CPL];
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            x[c] = active ? load_val<T>(kr + c) : 0.f;
            g[s][c] = active ? load_val<T>(gr + c) : 0.f;
            sum += x[c];
        }
        const float mean = wave_sum(sum) * (1.0f / DI);
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float dx = active ? x[c] - mean : 0.f;
            sq += dx * dx;
        }
        const float var = wave_sum(sq) * (1.0f / DI);
        const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[s][c] = (x[c] - mean) * rstd * wv[c] + bv[c];
    }
    if (!active) return;

    uint16_t outv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float m = g[0][c];
#pragma unroll
        for (int s = 1; s < KP; ++s) m = fmaxf(m, g[s][c]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int s = 0; s < KP; ++s) {
            const float e = expf(g[s][c] - m);
            den += e;
            num += e * y[s][c];
        }
        outv[c] = (uint16_t)f32_to_bf16_rne(num / den);
    }
    uint16_t* dst = pools + (pool_base[b] + p) * (int64_t)DI + c0;
    if constexpr (CPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)outv[0] | ((uint32_t)outv[1] << 16);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) dst[c] = outv[c];
    }
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_index_pools(const dsa_dims& d, const void* k, const void* gate, int dtype,
                              const float* ln_w, const float* ln_b, const dsa_seqs& seqs,
                              int32_t num_seqs, const int32_t* pool_begin,
                              const int32_t* pool_end, int32_t max_pools, uint16_t* pools,
                              hipStream_t s) {
    if (max_pools <= 0 || num_seqs <= 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(max_pools, 4), (unsigned)num_seqs), block(256);
#define DSA_POOLS(DI, T)                                                                          \
    hipLaunchKernelGGL((dsa::k_index_pools<DI, T>), grid, block, 0, s, (const T*)k, (const T*)gate, \
                       ln_w, ln_b, d.ln_eps, seqs.first_valid, seqs.tok_base, seqs.pool_base,      \
                       pool_begin, pool_end, pools)
    if (d.idx_dim == 128) {
        if (dtype == DSA_F32) DSA_POOLS(128, float); else DSA_POOLS(128, uint16_t);
    } else {
        if (dtype == DSA_F32) DSA_POOLS(32, float); else DSA_POOLS(32, uint16_t);
    }
#undef DSA_POOLS
    return hipGetLastError();
}

}  // namespace dsa_host
