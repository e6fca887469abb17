// store_int8: one latent row -> one INT8 cache row ([Kernels] Included:
// D int8 codes, the fp32 scale, zero padding to row_bytes).
//
// One wave per row.  Each lane owns D/64 consecutive values, so a 512-value
// bf16 row is one 16-byte load per lane and one 8-byte store per lane, fully
// coalesced.  The row's amax is a wave max; the scale and the codes use IEEE
// fp32 division (this file is built with correctly rounded fp32 divide) and
// v_rndne_f32 (round half to even).
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

template <int BYTES>
struct Bytes;
template <> struct Bytes<2>  { typedef uint16_t T; };
template <> struct Bytes<4>  { typedef uint32_t T; };
template <> struct Bytes<8>  { typedef u32x2 T; };
template <> struct Bytes<16> { typedef u32x4 T; };

template <int D, bool IN_F32>
__global__ __launch_bounds__(256) void k_store_int8(const void* __restrict__ latent, int64_t n,
                                                     int64_t ld, const int64_t* __restrict__ slots,
                                                     int8_t* __restrict__ cache, int row_bytes) {
    constexpr int VPL = D / 64;                       // values per lane
    constexpr int ESZ = IN_F32 ? 4 : 2;
    static_assert(D % 64 == 0 && VPL <= 16, "unsupported row width");
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const int64_t slot = slots[i];
    if (slot < 0) return;

    float x[VPL];
    {
        constexpr int NB = VPL * ESZ;                 // bytes per lane
        constexpr int PB = NB >= 16 ? 16 : NB;        // bytes per load
        typedef typename Bytes<PB>::T V;
        V raw[NB / PB];
        const char* src = reinterpret_cast<const char*>(latent) + (i * ld + lane * VPL) * ESZ;
#pragma unroll
        for (int c = 0; c < NB / PB; ++c) raw[c] = *reinterpret_cast<const V*>(src + c * PB);
        if constexpr (IN_F32) {
            const float* pv = reinterpret_cast<const float*>(raw);
#pragma unroll
            for (int e = 0; e < VPL; ++e) x[e] = pv[e];
        } else {
            const uint16_t* pv = reinterpret_cast<const uint16_t*>(raw);
#pragma unroll
            for (int e = 0; e < VPL; ++e) x[e] = bf16_to_f32(pv[e]);
        }
    }

    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = wave_max(amax);
    const float s = fmaxf(amax, 1e-4f) / 127.0f;

    uint8_t codes[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) {
        float r = rintf(x[e] / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        codes[e] = (uint8_t)(int8_t)(int)r;
    }
    int8_t* row = cache + slot * (int64_t)row_bytes;
    typedef typename Bytes<(VPL >= 2 ? VPL : 2)>::T CV;
    if constexpr (VPL >= 2) {
        CV cv;
        __builtin_memcpy(&cv, codes, VPL);
        *reinterpret_cast<CV*>(row + lane * VPL) = cv;
    } else {
        row[lane] = (int8_t)codes[0];
    }
    // Tail: fp32 scale then zeros, written in 16-byte pieces (row_bytes - D is a multiple of 16).
    const int tail_chunks = (row_bytes - D) >> 4;
    if (lane < tail_chunks) {
        u32x4 t = {lane == 0 ? __float_as_uint(s) : 0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(row + D + lane * 16) = t;
    }
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
