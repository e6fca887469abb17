// Shared device helpers for the gfx950 DSA kernels (wave64, MFMA, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 to packed bf16 (a in the low half), rounded to nearest even by
// the hardware's packed conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// x as bf16 hi + lo pairs for two values: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = f32x2_to_bf16x2(x0, x1);
    lo = f32x2_to_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 4 INT8 codes -> bf16 of (code + 128), 0..255, exact: one byte-to-float
// conversion per code (v_cvt_f32_ubyteN) and the upper halves packed.
__device__ __forceinline__ void biased4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const float f0 = (float)(u & 0xFFu);
    const float f1 = (float)((u >> 8) & 0xFFu);
    const float f2 = (float)((u >> 16) & 0xFFu);
    const float f3 = (float)(u >> 24);
    lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// max(x, 0) as one integer max on the bits: a value with the sign bit set
// (-0 included) gives +0, any other passes.  For a number this is the ReLU;
// fmaxf would first canonicalise an operand the compiler cannot prove
// canonical (an MFMA result), one more instruction per value.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// 8 INT8 codes (two words) -> 8 bf16 of (code + 128).
__device__ __forceinline__ u32x4 codes8_to_biased_bf16(uint32_t a, uint32_t b) {
    uint32_t r0, r1, r2, r3;
    biased4_to_bf16(a, r0, r1);
    biased4_to_bf16(b, r2, r3);
    return u32x4{r0, r1, r2, r3};
}

// ---------------------------------------------------------------- wave reductions
// Butterfly reductions over the 64 lanes of a wave; every lane gets the result
// and the combination order is fixed, so results are deterministic.

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Cross-half sums by gfx950's lane swaps (v_permlane32_swap_b32 trades the
// upper 32 lanes of one register with the lower 32 of another, 16-swap the
// odd and even 16-lane rows), no trip through the LDS pipe.  add_swap32(a, b):
// lanes 0..31 get a + a of lane l + 32, lanes 32..63 b + b of lane l - 32;
// add_swap16 the same across rows (lane l ^ 16).  Each sum adds the same two
// values in both lanes, so the results are those of the xor shuffles.
__device__ __forceinline__ float add_swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float add_swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------- DPP wave scans (integers)
// Inclusive scans over the 64 lanes with row shifts and row broadcasts: a
// handful of VALU operations instead of cross-lane shuffles through the LDS
// pipe.  Lanes whose source lies outside the row read the identity.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t identity) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROW_MASK, 0xF, false);
}

template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x, uint32_t identity, Op op) {
    x = op(x, dpp_u32<0x111, 0xF>(x, identity));      // row_shr:1
    x = op(x, dpp_u32<0x112, 0xF>(x, identity));      // row_shr:2
    x = op(x, dpp_u32<0x114, 0xF>(x, identity));      // row_shr:4
    x = op(x, dpp_u32<0x118, 0xF>(x, identity));      // row_shr:8
    x = op(x, dpp_u32<0x142, 0xA>(x, identity));      // row_bcast:15 into rows 1 and 3
    x = op(x, dpp_u32<0x143, 0xC>(x, identity));      // row_bcast:31 into rows 2 and 3
    return x;
}

// Max and sum over each row of 16 lanes, every lane of the row getting the
// result: a butterfly of DPP moves (lane ^ 1 and lane ^ 2 within quads, then
// the row's half mirror and mirror, which pair quads and halves) instead of
// cross-lane shuffles through the LDS pipe.  Each step adds a pair of lanes in
// both of them (the same two values), so every lane gets the same bits, the
// bits the xor-1, 2, 4, 8 shuffle butterfly gives.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f32<0xB1>(x));                   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f32<0x4E>(x));                   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f32<0x141>(x));                  // row_half_mirror
    return fmaxf(x, dpp_f32<0x140>(x));               // row_mirror
}

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    return x + dpp_f32<0x140>(x);
}

// Max and sum over all 64 lanes, every lane getting the result: the row
// butterflies above, then the lane swaps across rows and halves.
__device__ __forceinline__ float wave_allmax(float x) {
    x = row16_max(x);
    x = max_swap16(x, x);
    return max_swap32(x, x);
}

__device__ __forceinline__ float wave_allsum(float x) {
    x = row16_sum(x);
    x = add_swap16(x, x);
    return add_swap32(x, x);
}

// Inclusive sum within each row of 16 lanes (the first four steps above).
__device__ __forceinline__ uint32_t row_incl_sum_u32(uint32_t x) {
    x += dpp_u32<0x111, 0xF>(x, 0u);
    x += dpp_u32<0x112, 0xF>(x, 0u);
    x += dpp_u32<0x114, 0xF>(x, 0u);
    x += dpp_u32<0x118, 0xF>(x, 0u);
    return x;
}

__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t x) {
    return wave_incl_scan_u32(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    return __builtin_amdgcn_readlane(
        wave_incl_scan_u32(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    return __builtin_amdgcn_readlane(
        wave_incl_scan_u32(x, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; }), 63);
}

// ---------------------------------------------------------------- ordering keys
// Order-preserving map from fp32 to uint32 (larger float -> larger key),
// with -0 mapped onto +0 so the two compare equal.

__device__ __forceinline__ uint32_t f32_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: lane l holds A row (l % 16) and B column (l % 16),
// 8 k-values each for k-group (l / 16); D lane l holds column (l % 16), rows
// 4 * (l / 16) + i for i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: lane l holds A row (l % 32) and B column (l % 32),
// 8 k-values each for k-group (l / 32); D lane l holds column (l % 32), rows
// 8 * (r / 4) + 4 * (l / 32) + (r % 4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- barriers

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the compiler drain every outstanding global load before
// the barrier and so defeats register prefetching; none of these kernels
// exchange global memory between the waves of a workgroup.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Set bits of a wave mask in the lanes below this one (v_mbcnt: no per-lane
// mask has to be built or kept).
__device__ __forceinline__ int popc_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// A value every lane of the wave holds, moved to SGPRs (the compiler cannot
// always prove that a value read from LDS or derived from threadIdx is uniform).
__device__ __forceinline__ int uniform32(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// Raw buffer descriptor over [base, base + bytes) (both wave-uniform).  Loads
// through it take the base from SGPRs and a 32-bit lane offset; lane offsets
// past `bytes` read zero, but the SGPR offset is outside that check, so
// callers keep every access in bounds themselves.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    void* b = reinterpret_cast<void*>(uniform64(reinterpret_cast<uint64_t>(base)));
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, uniform32((int)bytes), 0x00020000);
}
// voff: the lane's byte offset; soff: a wave-uniform byte offset (SGPR).
__device__ __forceinline__ u32x4 ld_buf128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Orders LDS writes of this wave before its later LDS reads of other lanes'
// entries (no workgroup barrier).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// ---------------------------------------------------------------- block scans

// Exclusive prefix sum of one uint32 per thread over a block of NT threads.
// `sh` must hold NT / 64 + 1 entries.  Returns the exclusive prefix; *total
// receives the block total.  Waves scan with DPP; wave totals go through LDS
// once and every thread adds the totals of the waves before its own.
// Contains two LDS barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_sum_u32(v);
    if (lane == 63) sh[wave] = x;
    lds_barrier();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t tw = sh[w];
        before += w < wave ? tw : 0u;
        all += tw;
    }
    *total = all;
    lds_barrier();
    return before + x - v;
}

}  // namespace dsa

namespace dsa {
// Size of the fixed device array behind dsa_sparse_mla_noalloc (split partials).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
}  // namespace dsa

// Host-side helpers shared by the launchers.
namespace dsa_host {

struct DeviceInfo {
    int cu_count;
    size_t max_lds_per_block;
};

// Cached per device; never allocates device memory.
DeviceInfo device_info();

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dsa_host
