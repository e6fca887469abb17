// store_int8: one latent row -> one INT8 cache row per wave (the row code is
// store_int8_row, shared with the single-launch append).
#include "dsa_common.h"
#include "dsa_launch.h"
#include "new_tokens.h"

namespace dsa {

template <int D, bool IN_F32>
__global__ __launch_bounds__(256) void k_store_int8(const void* __restrict__ latent, int64_t n,
                                                     int64_t ld, const int64_t* __restrict__ slots,
                                                     int8_t* __restrict__ cache, int row_bytes) {
    store_int8_row<D, IN_F32>(latent, n, ld, slots, cache, row_bytes, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_store_int8(const dsa_dims& d, const void* latent, int dtype, int64_t n,
                             int64_t ld, const int64_t* slots, int8_t* cache, hipStream_t s) {
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(n, 4)), block(256);
    const bool f32 = dtype == DSA_F32;
    if (d.latent_dim == 512) {
        if (f32) hipLaunchKernelGGL((dsa::k_store_int8<512, true>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
        else     hipLaunchKernelGGL((dsa::k_store_int8<512, false>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
    } else if (d.latent_dim == 256) {
        if (f32) hipLaunchKernelGGL((dsa::k_store_int8<256, true>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
        else     hipLaunchKernelGGL((dsa::k_store_int8<256, false>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
    } else if (d.latent_dim == 128) {
        if (f32) hipLaunchKernelGGL((dsa::k_store_int8<128, true>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
        else     hipLaunchKernelGGL((dsa::k_store_int8<128, false>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
    } else {  // 64 (validated by the caller)
        if (f32) hipLaunchKernelGGL((dsa::k_store_int8<64, true>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
        else     hipLaunchKernelGGL((dsa::k_store_int8<64, false>), grid, block, 0, s, latent, n, ld, slots, cache, d.row_bytes);
    }
    return hipGetLastError();
}

}  // namespace dsa_host
