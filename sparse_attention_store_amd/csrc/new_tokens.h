// Device code for a step's new tokens, shared by the standalone kernels and
// the single-launch append:
//   store_int8_row -- one latent row -> one INT8 cache row ([Kernels]
//     Included: D int8 codes, the fp32 scale, zero padding to row_bytes).
//     Each lane owns D/64 consecutive values, so a 512-value bf16 row is one
//     16-byte load per lane and one 8-byte store per lane, fully coalesced.
//     The row's amax is a wave max; the scale and the codes use IEEE fp32
//     division (the library is built with correctly rounded fp32 divide) and
//     v_rndne_f32 (round half to even).
//   index_pool_row -- one kpool-token pool of LayerNorm'd indexer keys,
//     weighted by a per-channel softmax over the pool slots ([Ref] Traps:
//     LayerNorm with bias, softmax over the slot axis, pools from the first
//     valid token, full pools only; Functions: pool_states, layer_norm).  A
//     lane owns idx_dim/64 channels (2 for 128), reads the kpool token rows
//     of k and gate (4 x 256 B each per pool, coalesced), takes mean and
//     biased variance of each token row with two wave sums, and does the slot
//     softmax in registers: the softmax runs along the slot axis of a fixed
//     channel, so it needs no cross-lane step.
#pragma once
#include "dsa_common.h"

namespace dsa {

template <int BYTES>
struct Bytes;
template <> struct Bytes<2>  { typedef uint16_t T; };
template <> struct Bytes<4>  { typedef uint32_t T; };
template <> struct Bytes<8>  { typedef u32x2 T; };
template <> struct Bytes<16> { typedef u32x4 T; };

// Latent row i -> its cache row (one wave; every lane of the wave calls it).
template <int D, bool IN_F32>
__device__ __forceinline__ void store_int8_row(const void* __restrict__ latent, int64_t n, int64_t ld,
                                               const int64_t* __restrict__ slots, int8_t* __restrict__ cache,
                                               int row_bytes, int64_t i) {
    constexpr int VPL = D / 64;                       // values per lane
    constexpr int ESZ = IN_F32 ? 4 : 2;
    static_assert(D % 64 == 0 && VPL <= 16, "unsupported row width");
    const int lane = threadIdx.x & 63;
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

template <typename T>
__device__ __forceinline__ float load_val(const T* p);
template <> __device__ __forceinline__ float load_val<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_val<float>(const float* p) { return *p; }

// Pool pool_begin[b] + j of sequence b, if below pool_end[b] (one wave;
// every lane of the wave calls it).
template <int DI, typename T>
__device__ __forceinline__ void index_pool_row(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end,
    uint16_t* __restrict__ pools, int b, int j) {
    constexpr int KP = 4;
    constexpr int CPL = DI >= 64 ? DI / 64 : 1;       // channels per lane
    const int lane = threadIdx.x & 63;
    const int p = pool_begin[b] + j;
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
