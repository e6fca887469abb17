// index_pools: one wave per completed pool (the pool code is index_pool_row,
// shared with the single-launch append).
#include "dsa_common.h"
#include "dsa_launch.h"
#include "new_tokens.h"

namespace dsa {

template <int DI, typename T>
__global__ __launch_bounds__(256) void k_index_pools(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end,
    uint16_t* __restrict__ pools) {
    index_pool_row<DI, T>(k, gate, ln_w, ln_b, eps, first_valid, tok_base, pool_base, pool_begin, pool_end, pools,
                          blockIdx.y, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// The INT8 form ([Flash] What is quantized: INT8 indexer cache with a
// per-row fp32 scale): the same pools, quantised per row.
template <int DI, typename T>
__global__ __launch_bounds__(256) void k_index_pools_int8(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end, PoolDst dst) {
    index_pool_row_int8<DI, T>(k, gate, ln_w, ln_b, eps, first_valid, tok_base, pool_base, pool_begin, pool_end,
                               dst, blockIdx.y, blockIdx.x * 4 + (threadIdx.x >> 6));
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_index_pools_int8(const dsa_dims& d, const void* k, const void* gate, int dtype,
                                   const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                   const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                   int8_t* codes, float* scales, float* pools_f32, hipStream_t s) {
    if (max_pools <= 0 || num_seqs <= 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(max_pools, 4), (unsigned)num_seqs), block(256);
    const dsa::PoolDst dst{nullptr, codes, scales, pools_f32};
#define DSA_POOLS8(DI, T)                                                                               \
    hipLaunchKernelGGL((dsa::k_index_pools_int8<DI, T>), grid, block, 0, s, (const T*)k, (const T*)gate,  \
                       ln_w, ln_b, d.ln_eps, seqs.first_valid, seqs.tok_base, seqs.pool_base, pool_begin, \
                       pool_end, dst)
    if (d.idx_dim == 128) {
        if (dtype == DSA_F32) DSA_POOLS8(128, float); else DSA_POOLS8(128, uint16_t);
    } else {
        if (dtype == DSA_F32) DSA_POOLS8(32, float); else DSA_POOLS8(32, uint16_t);
    }
#undef DSA_POOLS8
    return hipGetLastError();
}

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
