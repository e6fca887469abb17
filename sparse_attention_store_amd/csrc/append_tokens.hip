// append_tokens: a step's new tokens in one launch -- their INT8 cache rows
// (store_int8_row) and the pools they complete (index_pool_row), the same
// device code as the standalone store_int8 and index_pools kernels.
// Workgroups [0, pool_blocks) build pools, 4 per workgroup (blockIdx ->
// (sequence, block of 4 pools)); the remaining workgroups store rows, 4 per
// workgroup.  The two kinds of work read and write disjoint buffers, so they
// need no ordering between them; both are a few dependent loads and a store
// per wave, so one launch costs what the slower of them does.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "new_tokens.h"

namespace dsa {

template <int D, int DI, typename T>
__global__ __launch_bounds__(256) void k_append_tokens(
    const void* __restrict__ latent, int64_t n, int64_t ld, const int64_t* __restrict__ slots,
    int8_t* __restrict__ cache, int row_bytes, const T* __restrict__ k, const T* __restrict__ gate,
    const float* __restrict__ ln_w, const float* __restrict__ ln_b, float eps,
    const int32_t* __restrict__ first_valid, const int64_t* __restrict__ tok_base,
    const int64_t* __restrict__ pool_base, const int32_t* __restrict__ pool_begin,
    const int32_t* __restrict__ pool_end, uint16_t* __restrict__ pools, int pool_bx, int pool_blocks) {
    const int wave = threadIdx.x >> 6;
    const int blk = (int)blockIdx.x;
    if (blk < pool_blocks) {
        index_pool_row<DI, T>(k, gate, ln_w, ln_b, eps, first_valid, tok_base, pool_base, pool_begin, pool_end,
                              pools, blk / pool_bx, (blk % pool_bx) * 4 + wave);
    } else {
        store_int8_row<D, std::is_same<T, float>::value>(latent, n, ld, slots, cache, row_bytes,
                                                         (int64_t)(blk - pool_blocks) * 4 + wave);
    }
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_append_tokens(const dsa_dims& d, int dtype, const void* latent, int64_t n, int64_t ld,
                                const int64_t* slots, int8_t* cache, const void* k, const void* gate,
                                const float* ln_w, const float* ln_b, const dsa_seqs& seqs, int32_t num_seqs,
                                const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                                uint16_t* pools, hipStream_t s) {
    const int pool_bx = max_pools > 0 && num_seqs > 0 ? (int)cdiv(max_pools, 4) : 0;
    const int64_t pool_blocks = (int64_t)pool_bx * (pool_bx ? num_seqs : 0);
    const int64_t blocks = pool_blocks + cdiv(n, 4);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(256);
#define DSA_APPEND(D, DI, T)                                                                              \
    hipLaunchKernelGGL((dsa::k_append_tokens<D, DI, T>), grid, block, 0, s, latent, n, ld, slots, cache,     \
                       d.row_bytes, (const T*)k, (const T*)gate, ln_w, ln_b, d.ln_eps, seqs.first_valid,     \
                       seqs.tok_base, seqs.pool_base, pool_begin, pool_end, pools, pool_bx ? pool_bx : 1,    \
                       (int)pool_blocks)
#define DSA_APPEND_DI(D, T)                                \
    if (d.idx_dim == 128) DSA_APPEND(D, 128, T);           \
    else DSA_APPEND(D, 32, T)
#define DSA_APPEND_T(D)                                    \
    if (dtype == DSA_F32) { DSA_APPEND_DI(D, float); }     \
    else { DSA_APPEND_DI(D, uint16_t); }
    switch (d.latent_dim) {
        case 512: DSA_APPEND_T(512); break;
        case 256: DSA_APPEND_T(256); break;
        case 128: DSA_APPEND_T(128); break;
        default: DSA_APPEND_T(64); break;   // 64 (validated by the caller)
    }
#undef DSA_APPEND_T
#undef DSA_APPEND_DI
#undef DSA_APPEND
    return hipGetLastError();
}

}  // namespace dsa_host
