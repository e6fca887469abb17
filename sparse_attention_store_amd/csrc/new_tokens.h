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

// One pool's inputs: this lane's channels of the kpool token rows of k and
// gate, from token row tok0 on.
template <int DI, typename T>
struct PoolIn {
    static constexpr int KP = 4;
    static constexpr int CPL = DI >= 64 ? DI / 64 : 1;       // channels per lane
    float x[KP][CPL], g[KP][CPL];
};

template <int DI, typename T>
__device__ __forceinline__ void pool_inputs(const T* __restrict__ k, const T* __restrict__ gate, int64_t tok0,
                                            PoolIn<DI, T>& in) {
    constexpr int KP = PoolIn<DI, T>::KP, CPL = PoolIn<DI, T>::CPL;
    const int lane = threadIdx.x & 63;
    const bool active = DI >= 64 || lane < DI;
    const int c0 = active ? lane * CPL : 0;
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        const T* kr = k + (tok0 + s) * DI + c0;
        const T* gr = gate + (tok0 + s) * DI + c0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            in.x[s][c] = active ? load_val<T>(kr + c) : 0.f;
            in.g[s][c] = active ? load_val<T>(gr + c) : 0.f;
        }
    }
}

// The same inputs for bf16 k and gate with idx_dim 128, kept as raw bit
// pairs (one 4-byte load per token row and lane): no conversion waits on the
// loads, so they can be issued long before the values are needed.
struct PoolRaw128 {
    uint32_t k[4], g[4];
};

// tok0 wave-uniform; the four rows of k and gate go through buffer
// descriptors over them, so a lane's address is one 32-bit offset.
__device__ __forceinline__ void pool_raw_load(const uint16_t* k, const uint16_t* gate, int64_t tok0, PoolRaw128& r) {
    const uint32_t off = (uint32_t)(threadIdx.x & 63) * 4u;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + tok0 * 128, 4 * 128 * 2);
    const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(gate + tok0 * 128, 4 * 128 * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        r.k[s] = __builtin_amdgcn_raw_buffer_load_b32(rk, off, (uint32_t)(256 * s), 0);
        r.g[s] = __builtin_amdgcn_raw_buffer_load_b32(rg, off, (uint32_t)(256 * s), 0);
    }
}

__device__ __forceinline__ void pool_raw_in(const PoolRaw128& r, PoolIn<128, uint16_t>& in) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        in.x[s][0] = __uint_as_float(r.k[s] << 16);
        in.x[s][1] = __uint_as_float(r.k[s] & 0xFFFF0000u);
        in.g[s][0] = __uint_as_float(r.g[s] << 16);
        in.g[s][1] = __uint_as_float(r.g[s] & 0xFFFF0000u);
    }
}

// The pool's values at this lane's channels (bf16, round to nearest even):
// LayerNorm of each token row, then the slot softmax.  Every lane of the wave
// calls it (wave sums); lanes past DI get zeros.
// Contraction is off and the fused multiply-adds are written out, so every
// kernel that inlines this produces the same bits.
template <int DI, typename T>
__device__ __forceinline__ void pool_values(const PoolIn<DI, T>& in, const float* __restrict__ ln_w,
                                            const float* __restrict__ ln_b, float eps,
                                            uint16_t (&outv)[PoolIn<DI, T>::CPL]) {
#pragma clang fp contract(off)
    constexpr int KP = PoolIn<DI, T>::KP, CPL = PoolIn<DI, T>::CPL;
    const int lane = threadIdx.x & 63;
    const bool active = DI >= 64 || lane < DI;
    const int c0 = active ? lane * CPL : 0;
    // ln_w / ln_b through buffer descriptors: the lane's offset is a 32-bit
    // value, cheap to recompute, so no per-lane pointer is kept live.
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(ln_w, DI * 4), rb = buffer_rsrc(ln_b, DI * 4);
    float wv[CPL], bv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        wv[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(c0 + c) * 4u, 0, 0));
        bv[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(c0 + c) * 4u, 0, 0));
    }
    float y[KP][CPL];
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) sum += in.x[s][c];
        const float mean = wave_sum(sum) * (1.0f / DI);
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float dx = active ? in.x[s][c] - mean : 0.f;
            sq = __builtin_fmaf(dx, dx, sq);
        }
        const float var = wave_sum(sq) * (1.0f / DI);
        const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[s][c] = __builtin_fmaf((in.x[s][c] - mean) * rstd, wv[c], bv[c]);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float m = in.g[0][c];
#pragma unroll
        for (int s = 1; s < KP; ++s) m = fmaxf(m, in.g[s][c]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int s = 0; s < KP; ++s) {
            const float e = expf(in.g[s][c] - m);
            den += e;
            num = __builtin_fmaf(e, y[s][c], num);
        }
        outv[c] = active ? (uint16_t)f32_to_bf16_rne(num / den) : (uint16_t)0;
    }
}

// The same values in fp32, before any rounding (the INT8 pool form quantises
// these).  The arithmetic is pool_values' up to its final rounding, written
// out again rather than shared so that the bf16 kernels' code is unchanged.
template <int DI, typename T>
__device__ __forceinline__ void pool_values_f32(const PoolIn<DI, T>& in, const float* __restrict__ ln_w,
                                                const float* __restrict__ ln_b, float eps,
                                                float (&outv)[PoolIn<DI, T>::CPL]) {
#pragma clang fp contract(off)
    constexpr int KP = PoolIn<DI, T>::KP, CPL = PoolIn<DI, T>::CPL;
    const int lane = threadIdx.x & 63;
    const bool active = DI >= 64 || lane < DI;
    const int c0 = active ? lane * CPL : 0;
    // ln_w / ln_b through buffer descriptors: the lane's offset is a 32-bit
    // value, cheap to recompute, so no per-lane pointer is kept live.
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(ln_w, DI * 4), rb = buffer_rsrc(ln_b, DI * 4);
    float wv[CPL], bv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        wv[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(c0 + c) * 4u, 0, 0));
        bv[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(c0 + c) * 4u, 0, 0));
    }
    float y[KP][CPL];
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) sum += in.x[s][c];
        const float mean = wave_sum(sum) * (1.0f / DI);
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float dx = active ? in.x[s][c] - mean : 0.f;
            sq = __builtin_fmaf(dx, dx, sq);
        }
        const float var = wave_sum(sq) * (1.0f / DI);
        const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[s][c] = __builtin_fmaf((in.x[s][c] - mean) * rstd, wv[c], bv[c]);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float m = in.g[0][c];
#pragma unroll
        for (int s = 1; s < KP; ++s) m = fmaxf(m, in.g[s][c]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int s = 0; s < KP; ++s) {
            const float e = expf(in.g[s][c] - m);
            den += e;
            num = __builtin_fmaf(e, y[s][c], num);
        }
        outv[c] = active ? num / den : 0.f;
    }
}

// A pool's fp32 values as INT8 codes with one fp32 scale for the row ([Flash]
// What is quantized: the INT8 indexer cache, one scale per row), by the
// quantiser of the latent rows: amax over the row (a wave max; lanes past DI
// hold zeros), s = max(amax, 1e-4) / 127 (IEEE division), code =
// clamp(round_half_even(x / s), -127, 127).  Every lane of the wave calls it.
template <int CPL>
__device__ __forceinline__ float quantize_pool(const float (&f)[CPL], int8_t (&code)[CPL]) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) amax = fmaxf(amax, fabsf(f[c]));
    amax = wave_max(amax);
    const float s = fmaxf(amax, 1e-4f) / 127.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float r = rintf(f[c] / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        code[c] = (int8_t)(int)r;
    }
    return s;
}

// Where built pools go: bf16 rows, or INT8 code rows with a scale per row
// (and, when f32 is set, the fp32 values before quantisation).
struct PoolDst {
    uint16_t* bf16;    // [*, DI] bf16, or null for the INT8 form
    int8_t* codes;     // [*, DI] int8 (INT8 form)
    float* scales;     // [*] fp32 (INT8 form)
    float* f32;        // [*, DI] fp32 or null (INT8 form only)
};

// Pool pool_begin[b] + j of sequence b, if below pool_end[b] (one wave;
// every lane of the wave calls it).
template <int DI, typename T>
__device__ __forceinline__ void index_pool_row(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end,
    uint16_t* __restrict__ pools, int b, int j) {
    constexpr int CPL = PoolIn<DI, T>::CPL;
    const int lane = threadIdx.x & 63;
    const int p = pool_begin[b] + j;
    if (p >= pool_end[b]) return;
    const int64_t tok0 = tok_base[b] + first_valid[b] + 4 * (int64_t)p;
    PoolIn<DI, T> in;
    pool_inputs<DI, T>(k, gate, tok0, in);
    uint16_t outv[CPL];
    pool_values<DI, T>(in, ln_w, ln_b, eps, outv);
    if (!(DI >= 64 || lane < DI)) return;
    uint16_t* dst = pools + (pool_base[b] + p) * (int64_t)DI + lane * CPL;
    if constexpr (CPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)outv[0] | ((uint32_t)outv[1] << 16);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) dst[c] = outv[c];
    }
}

// The same pool in the INT8 form: codes, its scale, and the fp32 values when
// dst.f32 is set.
template <int DI, typename T>
__device__ __forceinline__ void index_pool_row_int8(
    const T* __restrict__ k, const T* __restrict__ gate, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ tok_base, const int64_t* __restrict__ pool_base,
    const int32_t* __restrict__ pool_begin, const int32_t* __restrict__ pool_end, const PoolDst& dst, int b,
    int j) {
    constexpr int CPL = PoolIn<DI, T>::CPL;
    const int lane = threadIdx.x & 63;
    const int p = pool_begin[b] + j;
    if (p >= pool_end[b]) return;
    const int64_t tok0 = tok_base[b] + first_valid[b] + 4 * (int64_t)p;
    PoolIn<DI, T> in;
    pool_inputs<DI, T>(k, gate, tok0, in);
    float f[CPL];
    pool_values_f32<DI, T>(in, ln_w, ln_b, eps, f);
    int8_t code[CPL];
    const float s = quantize_pool<CPL>(f, code);
    const int64_t row = pool_base[b] + p;
    if (lane == 0) dst.scales[row] = s;
    if (!(DI >= 64 || lane < DI)) return;
    int8_t* cd = dst.codes + row * (int64_t)DI + lane * CPL;
    if constexpr (CPL == 2) {
        *reinterpret_cast<uint16_t*>(cd) = (uint16_t)((uint8_t)code[0] | ((uint32_t)(uint8_t)code[1] << 8));
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) cd[c] = code[c];
    }
    if (dst.f32) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) dst.f32[row * (int64_t)DI + lane * CPL + c] = f[c];
    }
}

}  // namespace dsa
