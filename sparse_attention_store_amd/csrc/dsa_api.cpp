// C ABI entry points: argument validation, dispatch, status codes.
// Only host-visible arguments are checked; device contents are trusted.
// Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "dsa.h"
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa_host {

DeviceInfo device_info() {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    static std::vector<bool> have;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) {
        cache.resize(dev + 1);
        have.resize(dev + 1, false);
    }
    if (!have[dev]) {
        DeviceInfo info{256, 160 * 1024};
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            info.cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
            if (prop.sharedMemPerBlock > 0) info.max_lds_per_block = prop.sharedMemPerBlock;
        }
        cache[dev] = info;
        have[dev] = true;
    }
    return cache[dev];
}

}  // namespace dsa_host

namespace {

using dsa_host::cdiv;

int check_dims(const dsa_dims* d) {
    if (!d) return DSA_ERR_NULL;
    if (d->idx_heads <= 0 || d->idx_dim <= 0 || d->kpool <= 0 || d->index_topk <= 0 ||
        d->out_width <= 0 || d->mla_heads <= 0 || d->latent_dim <= 0 || d->row_bytes <= 0 ||
        !(d->ln_eps >= 0.0f))
        return DSA_ERR_DIMS;
    if (d->index_topk % d->kpool != 0) return DSA_ERR_DIMS;
    if (d->row_bytes != (int)(((d->latent_dim + 4 + 15) / 16) * 16)) return DSA_ERR_DIMS;
    if (d->out_width < d->index_topk + d->kpool - 1) return DSA_ERR_WIDTH;
    return DSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_seqs(const dsa_seqs* s, int32_t num_seqs, bool need_row, bool need_tok, bool need_pool) {
    if (!s) return DSA_ERR_NULL;
    if (num_seqs <= 0) return DSA_ERR_SIZE;
    if (!s->first_valid) return DSA_ERR_NULL;
    if (need_row && !s->row_base) return DSA_ERR_NULL;
    if (need_tok && !s->tok_base) return DSA_ERR_NULL;
    if (need_pool && !s->pool_base) return DSA_ERR_NULL;
    return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
    switch (status) {
        case DSA_OK: return "ok";
        case DSA_ERR_NULL: return "a required pointer is NULL";
        case DSA_ERR_DIMS: return "inconsistent or non-positive dims";
        case DSA_ERR_DTYPE: return "dtype not accepted by this call";
        case DSA_ERR_ALIGN: return "pointer or leading dimension misaligned";
        case DSA_ERR_WIDTH: return "out_width < index_topk + kpool - 1";
        case DSA_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA_ERR_UNSUPPORTED: return "dims not supported by this build";
        case DSA_ERR_HIP: return "HIP runtime error";
        case DSA_ERR_SIZE: return "negative count or stride too small";
        case DSA_ERR_TIMEOUT: return "a wait inside the launch timed out; its results are invalid";
        case DSA_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int dsa_store_int8(const dsa_dims* dims, const void* latent, int latent_dtype, int64_t n,
                   int64_t ld, const int64_t* slots, int8_t* cache, int64_t cache_rows,
                   void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (n < 0 || cache_rows < 0) return DSA_ERR_SIZE;
    if (latent_dtype != DSA_F32 && latent_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    const int D = dims->latent_dim;
    if (D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_UNSUPPORTED;
    if (n == 0) return DSA_OK;
    if (!latent || !slots || !cache) return DSA_ERR_NULL;
    if (ld < D) return DSA_ERR_SIZE;
    const size_t esz = latent_dtype == DSA_F32 ? 4 : 2;
    if (!aligned(latent, 16) || (ld * esz) % 16 != 0 || !aligned(cache, 16)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_store_int8(*dims, latent, latent_dtype, n, ld, slots, cache,
                                                  as_stream(stream)));
}

int dsa_index_pools(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype,
                    const float* ln_w, const float* ln_b, const dsa_seqs* seqs, int32_t num_seqs,
                    const int32_t* pool_begin, const int32_t* pool_end, int32_t max_pools,
                    uint16_t* pools, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (kg_dtype != DSA_F32 && kg_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dims->kpool != 4 || (dims->idx_dim != 128 && dims->idx_dim != 32)) return DSA_ERR_UNSUPPORTED;
    if (max_pools < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, false, true, true);
    if (st) return st;
    if (num_seqs > 65535) return DSA_ERR_SIZE;
    if (max_pools == 0) return DSA_OK;
    if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end || !pools) return DSA_ERR_NULL;
    if (!aligned(k, 4) || !aligned(gate, 4) || !aligned(pools, 4)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_index_pools(*dims, k, gate, kg_dtype, ln_w, ln_b, *seqs, num_seqs,
                                                   pool_begin, pool_end, max_pools, pools,
                                                   as_stream(stream)));
}

int dsa_append_tokens(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                      const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                      const void* gate, const float* ln_w, const float* ln_b, const dsa_seqs* seqs,
                      int32_t num_seqs, const int32_t* pool_begin, const int32_t* pool_end,
                      int32_t max_pools, uint16_t* pools, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
    const int D = dims->latent_dim;
    if (D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_UNSUPPORTED;
    if (dims->kpool != 4 || (dims->idx_dim != 128 && dims->idx_dim != 32)) return DSA_ERR_UNSUPPORTED;
    if (n < 0 || cache_rows < 0 || max_pools < 0) return DSA_ERR_SIZE;
    if (n > 0) {
        if (!latent || !slots || !cache) return DSA_ERR_NULL;
        if (ld < D) return DSA_ERR_SIZE;
        const size_t esz = dtype == DSA_F32 ? 4 : 2;
        if (!aligned(latent, 16) || (ld * esz) % 16 != 0 || !aligned(cache, 16)) return DSA_ERR_ALIGN;
    }
    if (max_pools > 0) {
        st = check_seqs(seqs, num_seqs, false, true, true);
        if (st) return st;
        if (num_seqs > 65535) return DSA_ERR_SIZE;
        if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end || !pools) return DSA_ERR_NULL;
        if (!aligned(k, 4) || !aligned(gate, 4) || !aligned(pools, 4)) return DSA_ERR_ALIGN;
    }
    if (n == 0 && max_pools == 0) return DSA_OK;
    const dsa_seqs none{};
    return hip_status(dsa_host::launch_append_tokens(*dims, dtype, latent, n, ld, slots, cache, k, gate, ln_w,
                                                     ln_b, max_pools > 0 ? *seqs : none,
                                                     max_pools > 0 ? num_seqs : 0, pool_begin, pool_end,
                                                     max_pools, pools, as_stream(stream)));
}

int dsa_index_scores(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                     const uint16_t* pools, const dsa_seqs* seqs, int32_t num_seqs,
                     const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                     float* scores, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (dims->kpool != 4) return DSA_ERR_UNSUPPORTED;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, false, false, true);
    if (st) return st;
    if (T == 0 || score_stride == 0) return DSA_OK;
    if (T > 65535 * 64) return DSA_ERR_SIZE;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(scores, 4)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_index_scores(*dims, q_idx, w, pools, *seqs, num_seqs, q_seq, q_pos, T,
                                                    score_stride, scores, as_stream(stream)));
}

size_t dsa_topk_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride) {
    if (check_dims(dims) != DSA_OK) return 0;
    return dsa_host::topk_workspace_bytes(*dims, T, score_stride);
}

static int topk_common(const dsa_dims* dims, const float* scores, int32_t score_stride,
                       const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                       void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    if (dims->kpool != 4 || !dsa_host::topk_supported(*dims, score_stride)) return DSA_ERR_UNSUPPORTED;
    st = check_seqs(seqs, num_seqs, indices != nullptr, false, false);
    if (st) return st;
    if (T == 0) return DSA_OK;
    if (T > 65535) return DSA_ERR_SIZE;
    if (!scores || !q_seq || !q_pos || (!pool_ids && !indices)) return DSA_ERR_NULL;
    const size_t need = dsa_host::topk_workspace_bytes(*dims, T, score_stride);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    }
    return hip_status(dsa_host::launch_topk(*dims, scores, score_stride, *seqs, q_seq, q_pos, T,
                                            pool_ids, indices, workspace, as_stream(stream)));
}

int dsa_topk_select(const dsa_dims* dims, const float* scores, int32_t score_stride,
                    const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                    const int32_t* q_pos, int32_t T, int32_t* pool_ids, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!pool_ids) return DSA_ERR_NULL;
    return topk_common(dims, scores, score_stride, seqs, num_seqs, q_seq, q_pos, T, pool_ids, nullptr,
                       workspace, workspace_bytes, stream);
}

int dsa_topk_select_expand(const dsa_dims* dims, const float* scores, int32_t score_stride,
                           const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!indices) return DSA_ERR_NULL;
    return topk_common(dims, scores, score_stride, seqs, num_seqs, q_seq, q_pos, T, pool_ids, indices,
                       workspace, workspace_bytes, stream);
}

size_t dsa_index_scores_select_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride) {
    if (check_dims(dims) != DSA_OK || T <= 0 || score_stride <= 0) return 0;
    if (dsa_host::scores_select_grouped(*dims, T, score_stride)) return dsa_host::scores_select_group_bytes(T);
    return dsa_host::topk_workspace_bytes(*dims, T, score_stride);
}

static int groups_common(const dsa_dims* dims, const dsa_seqs* seqs, int32_t num_seqs, int32_t T,
                         int32_t score_stride, void* workspace, size_t workspace_bytes, bool long_rows = true) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, true, false, true);
    if (st) return st;
    if (T > 0 && !(long_rows ? dsa_host::scores_select_grouped(*dims, T, score_stride)
                             : dsa_host::scores_lists_short(*dims, T, score_stride)))
        return DSA_ERR_UNSUPPORTED;
    if (T == 0 || score_stride == 0) return DSA_OK;
    if (!workspace || workspace_bytes < dsa_host::scores_select_group_bytes(T)) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

int dsa_index_scores_groups(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                            const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                            int32_t T, int32_t score_stride, float* scores, void* workspace, size_t workspace_bytes,
                            void* stream) {
    int st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st || T == 0 || score_stride == 0) return st;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_scores_with_groups(*dims, q_idx, w, pools, *seqs, num_seqs, q_seq, q_pos, T,
                                                          score_stride, scores, workspace, as_stream(stream)));
}

int dsa_append_scores_groups(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                             const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                             const void* gate, const float* ln_w, const float* ln_b, const int32_t* pool_begin,
                             const int32_t* pool_end, int32_t max_pools, uint16_t* pools, const uint16_t* q_idx,
                             const float* w, const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t T, int32_t score_stride, float* scores, void* workspace,
                             size_t workspace_bytes, void* stream) {
    // The new tokens' part: exactly what dsa_append_tokens checks.
    int st = check_dims(dims);
    if (st) return st;
    if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
    const int D = dims->latent_dim;
    if (D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_UNSUPPORTED;
    if (dims->kpool != 4 || (dims->idx_dim != 128 && dims->idx_dim != 32)) return DSA_ERR_UNSUPPORTED;
    if (n < 0 || cache_rows < 0 || max_pools < 0) return DSA_ERR_SIZE;
    if (n > 0) {
        if (!latent || !slots || !cache) return DSA_ERR_NULL;
        if (ld < D) return DSA_ERR_SIZE;
        const size_t esz = dtype == DSA_F32 ? 4 : 2;
        if (!aligned(latent, 16) || (ld * esz) % 16 != 0 || !aligned(cache, 16)) return DSA_ERR_ALIGN;
    }
    // The scoring part: exactly what dsa_index_scores_groups checks.
    st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st) return st;
    if (max_pools > 0) {
        st = check_seqs(seqs, num_seqs, false, true, true);
        if (st) return st;
        if (num_seqs > 65535) return DSA_ERR_SIZE;
        if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end || !pools) return DSA_ERR_NULL;
        if (!aligned(k, 4) || !aligned(gate, 4) || !aligned(pools, 4)) return DSA_ERR_ALIGN;
    }
    const bool scoring = T > 0 && score_stride > 0;
    if (scoring) {
        if (!q_idx || !w || !pools || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
        if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    }
    hipStream_t s = as_stream(stream);
    const dsa_seqs none{};
    if (!scoring || !dsa_host::append_scores_fused(*dims, dtype)) {
        if (n > 0 || max_pools > 0) {
            hipError_t e = dsa_host::launch_append_tokens(*dims, dtype, latent, n, ld, slots, cache, k, gate, ln_w,
                                                          ln_b, max_pools > 0 ? *seqs : none,
                                                          max_pools > 0 ? num_seqs : 0, pool_begin, pool_end,
                                                          max_pools, pools, s);
            if (e != hipSuccess) return DSA_ERR_HIP;
        }
        if (!scoring) return DSA_OK;
        return hip_status(dsa_host::launch_scores_with_groups(*dims, q_idx, w, pools, *seqs, num_seqs, q_seq, q_pos, T,
                                                              score_stride, scores, workspace, s));
    }
    return hip_status(dsa_host::launch_append_scores_groups(
        *dims, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, *seqs, num_seqs, pool_begin,
        pool_end, max_pools, pools, q_idx, w, q_seq, q_pos, T, score_stride, scores, workspace, s));
}

// ------------------------------------------------------------------ INT8 pool cache

int dsa_index_pools_int8(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype, const float* ln_w,
                         const float* ln_b, const dsa_seqs* seqs, int32_t num_seqs, const int32_t* pool_begin,
                         const int32_t* pool_end, int32_t max_pools, int8_t* pool_codes, float* pool_scales,
                         float* pools_f32, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (kg_dtype != DSA_F32 && kg_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dims->kpool != 4 || (dims->idx_dim != 128 && dims->idx_dim != 32)) return DSA_ERR_UNSUPPORTED;
    st = check_seqs(seqs, num_seqs, false, true, true);
    if (st) return st;
    if (max_pools < 0) return DSA_ERR_SIZE;
    if (max_pools == 0) return DSA_OK;
    if (num_seqs > 65535) return DSA_ERR_SIZE;
    if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end || !pool_codes || !pool_scales) return DSA_ERR_NULL;
    if (!aligned(pool_codes, 16) || !aligned(pool_scales, 4) || !aligned(pools_f32, 4)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_index_pools_int8(*dims, k, gate, kg_dtype, ln_w, ln_b, *seqs, num_seqs,
                                                        pool_begin, pool_end, max_pools, pool_codes, pool_scales,
                                                        pools_f32, as_stream(stream)));
}

static bool int8_scoring_supported(const dsa_dims* d, int32_t T) {
    return d->idx_heads == 32 && d->idx_dim == 128 && d->kpool == 4 && T <= 64;
}

int dsa_index_scores_int8(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const int8_t* pool_codes,
                          const float* pool_scales, const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                          const int32_t* q_pos, int32_t T, int32_t score_stride, float* scores, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, false, false, true);
    if (st) return st;
    if (!int8_scoring_supported(dims, T)) return DSA_ERR_UNSUPPORTED;
    if (T == 0 || score_stride == 0) return DSA_OK;
    if (!q_idx || !w || !pool_codes || !pool_scales || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(w, 16) || !aligned(pool_codes, 16) || !aligned(pool_scales, 4) ||
        !aligned(scores, 4))
        return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_index_scores_int8(*dims, q_idx, w, pool_codes, pool_scales, *seqs, num_seqs,
                                                         q_seq, q_pos, T, score_stride, scores, as_stream(stream)));
}

int dsa_index_scores_groups_int8(const dsa_dims* dims, const uint16_t* q_idx, const float* w,
                                 const int8_t* pool_codes, const float* pool_scales, const dsa_seqs* seqs,
                                 int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                                 int32_t score_stride, float* scores, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    int st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st || T == 0 || score_stride == 0) return st;
    if (!q_idx || !w || !pool_codes || !pool_scales || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(w, 16) || !aligned(pool_codes, 16) || !aligned(pool_scales, 4))
        return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_scores_with_groups_int8(*dims, q_idx, w, pool_codes, pool_scales, *seqs,
                                                               num_seqs, q_seq, q_pos, T, score_stride, scores,
                                                               workspace, as_stream(stream)));
}

int dsa_append_scores_groups_int8(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                                  const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                                  const void* gate, const float* ln_w, const float* ln_b, const int32_t* pool_begin,
                                  const int32_t* pool_end, int32_t max_pools, int8_t* pool_codes, float* pool_scales,
                                  const uint16_t* q_idx, const float* w, const dsa_seqs* seqs, int32_t num_seqs,
                                  const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                                  float* scores, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (dtype != DSA_BF16) return dtype == DSA_F32 ? DSA_ERR_UNSUPPORTED : DSA_ERR_DTYPE;
    const int D = dims->latent_dim;
    if (D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_UNSUPPORTED;
    if (n < 0 || cache_rows < 0 || max_pools < 0) return DSA_ERR_SIZE;
    if (n > 0) {
        if (!latent || !slots || !cache) return DSA_ERR_NULL;
        if (ld < D) return DSA_ERR_SIZE;
        if (!aligned(latent, 16) || (ld * 2) % 16 != 0 || !aligned(cache, 16)) return DSA_ERR_ALIGN;
    }
    st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st) return st;
    if (!int8_scoring_supported(dims, T)) return DSA_ERR_UNSUPPORTED;
    if (max_pools > 0) {
        st = check_seqs(seqs, num_seqs, false, true, true);
        if (st) return st;
        if (num_seqs > 65535) return DSA_ERR_SIZE;
        if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end) return DSA_ERR_NULL;
        if (!aligned(k, 4) || !aligned(gate, 4)) return DSA_ERR_ALIGN;
    }
    if (!pool_codes || !pool_scales) return DSA_ERR_NULL;
    if (!aligned(pool_codes, 16) || !aligned(pool_scales, 4)) return DSA_ERR_ALIGN;
    const bool scoring = T > 0 && score_stride > 0;
    if (scoring) {
        if (!q_idx || !w || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
        if (!aligned(q_idx, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    }
    if (!scoring && n == 0 && max_pools == 0) return DSA_OK;
    const dsa_seqs none{};
    return hip_status(dsa_host::launch_append_scores_groups_int8(
        *dims, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, num_seqs > 0 && seqs ? *seqs : none, num_seqs,
        pool_begin, pool_end, max_pools, pool_codes, pool_scales, q_idx, w, q_seq, q_pos, scoring ? T : 0,
        scoring ? score_stride : 0, scores, workspace, as_stream(stream)));
}

int dsa_append_scores_groups_shared(const dsa_dims* dims, int dtype, const void* latent, int64_t n, int64_t ld,
                                    const int64_t* slots, int8_t* cache, int64_t cache_rows, const void* k,
                                    const void* gate, const float* ln_w, const float* ln_b, const int32_t* pool_begin,
                                    const int32_t* pool_end, int32_t max_pools, void* pools, float* pool_scales,
                                    const uint16_t* q_idx, const float* w, const dsa_seqs* seqs, int32_t num_seqs,
                                    const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t score_stride,
                                    float* scores, void* workspace, size_t workspace_bytes, int32_t share,
                                    void* stream) {
    if (share < 1 || share > 4) return DSA_ERR_SIZE;
    if (share == 1) {
        if (pool_scales)
            return dsa_append_scores_groups_int8(dims, dtype, latent, n, ld, slots, cache, cache_rows, k, gate, ln_w,
                                                 ln_b, pool_begin, pool_end, max_pools,
                                                 reinterpret_cast<int8_t*>(pools), pool_scales, q_idx, w, seqs,
                                                 num_seqs, q_seq, q_pos, T, score_stride, scores, workspace,
                                                 workspace_bytes, stream);
        return dsa_append_scores_groups(dims, dtype, latent, n, ld, slots, cache, cache_rows, k, gate, ln_w, ln_b,
                                        pool_begin, pool_end, max_pools, reinterpret_cast<uint16_t*>(pools), q_idx,
                                        w, seqs, num_seqs, q_seq, q_pos, T, score_stride, scores, workspace,
                                        workspace_bytes, stream);
    }
    int st = check_dims(dims);
    if (st) return st;
    if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
    const int D = dims->latent_dim;
    if (D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_UNSUPPORTED;
    if (n < 0 || cache_rows < 0 || max_pools < 0) return DSA_ERR_SIZE;
    const bool tokens = n > 0 || max_pools > 0;
    if (tokens && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
    if (n > 0) {
        if (!latent || !slots || !cache) return DSA_ERR_NULL;
        if (ld < D) return DSA_ERR_SIZE;
        if (!aligned(latent, 16) || (ld * 2) % 16 != 0 || !aligned(cache, 16)) return DSA_ERR_ALIGN;
    }
    st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes, false);   // runs: 64-pool groups
    if (st) return st;
    if (!int8_scoring_supported(dims, T)) return DSA_ERR_UNSUPPORTED;
    if (max_pools > 0) {
        st = check_seqs(seqs, num_seqs, false, true, true);
        if (st) return st;
        if (num_seqs > 65535) return DSA_ERR_SIZE;
        if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end) return DSA_ERR_NULL;
        if (!aligned(k, 4) || !aligned(gate, 4)) return DSA_ERR_ALIGN;
    }
    if (!pools) return DSA_ERR_NULL;
    if (!aligned(pools, 16) || !aligned(pool_scales, 4)) return DSA_ERR_ALIGN;
    const bool scoring = T > 0 && score_stride > 0;
    if (scoring) {
        if (!q_idx || !w || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
        if (!aligned(q_idx, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    }
    if (!scoring && !tokens) return DSA_OK;
    const dsa_seqs none{};
    return hip_status(dsa_host::launch_append_scores_groups_runs(
        *dims, latent, n, ld, slots, cache, k, gate, ln_w, ln_b, num_seqs > 0 && seqs ? *seqs : none, num_seqs,
        pool_begin, pool_end, max_pools, pools, pool_scales, q_idx, w, q_seq, q_pos, scoring ? T : 0,
        scoring ? score_stride : 0, scores, workspace, share, as_stream(stream)));
}

// ------------------------------------------------------------------ paged caches

static int check_paged(const dsa_paged_seqs* s, int32_t num_seqs) {
    if (!s) return DSA_ERR_NULL;
    if (num_seqs <= 0 || s->table_stride <= 0) return DSA_ERR_SIZE;
    if (!s->first_valid || !s->block_table) return DSA_ERR_NULL;
    return DSA_OK;
}

int dsa_index_pools_paged(const dsa_dims* dims, const void* k, const void* gate, int kg_dtype, const float* ln_w,
                          const float* ln_b, const dsa_paged_seqs* seqs, int32_t num_seqs, const int32_t* pool_begin,
                          const int32_t* pool_end, int32_t max_pools, uint16_t* pools, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (kg_dtype != DSA_F32 && kg_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dims->kpool != 4 || (dims->idx_dim != 128 && dims->idx_dim != 32)) return DSA_ERR_UNSUPPORTED;
    st = check_paged(seqs, num_seqs);
    if (st) return st;
    if (max_pools < 0) return DSA_ERR_SIZE;
    if (max_pools == 0) return DSA_OK;
    if (num_seqs > 65535) return DSA_ERR_SIZE;
    if (!k || !gate || !ln_w || !ln_b || !pool_begin || !pool_end || !pools) return DSA_ERR_NULL;
    if (!aligned(pools, 4)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_index_pools_paged(*dims, k, gate, kg_dtype, ln_w, ln_b, seqs->first_valid,
                                                         seqs->block_table, seqs->table_stride, num_seqs, pool_begin,
                                                         pool_end, max_pools, pools, as_stream(stream)));
}

static int paged_groups_common(const dsa_dims* dims, const dsa_paged_seqs* seqs, int32_t num_seqs, int32_t T,
                               int32_t score_stride, void* workspace, size_t workspace_bytes) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    st = check_paged(seqs, num_seqs);
    if (st) return st;
    if (T > 0 && !dsa_host::scores_lists_short(*dims, T, score_stride)) return DSA_ERR_UNSUPPORTED;
    if (T == 0 || score_stride == 0) return DSA_OK;
    if (!workspace || workspace_bytes < dsa_host::scores_select_group_bytes(T)) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

int dsa_index_scores_groups_paged(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                                  const dsa_paged_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                                  const int32_t* q_pos, int32_t T, int32_t score_stride, float* scores,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    int st = paged_groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st || T == 0 || score_stride == 0) return st;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !scores) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_scores_with_groups_paged(*dims, q_idx, w, pools, seqs->first_valid,
                                                                seqs->block_table, seqs->table_stride, num_seqs,
                                                                q_seq, q_pos, T, score_stride, scores, workspace,
                                                                as_stream(stream)));
}

int dsa_topk_select_groups_paged(const dsa_dims* dims, const float* scores, int32_t score_stride,
                                 const dsa_paged_seqs* seqs, int32_t num_seqs, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t T, int32_t* pool_ids, int32_t* indices,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    int st = paged_groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st || T == 0 || score_stride == 0) return st;
    if (!scores || !q_seq || !q_pos || !indices) return DSA_ERR_NULL;
    return hip_status(dsa_host::launch_topk_groups_paged(*dims, scores, score_stride, seqs->first_valid,
                                                         seqs->block_table, seqs->table_stride, q_seq, q_pos, T,
                                                         pool_ids, indices, workspace, as_stream(stream)));
}

int dsa_time_next_scoring_launch(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return DSA_ERR_NULL;
    dsa_host::time_next_scoring_launch(reinterpret_cast<hipEvent_t>(start_event),
                                       reinterpret_cast<hipEvent_t>(stop_event));
    return DSA_OK;
}

int dsa_topk_select_groups(const dsa_dims* dims, const float* scores, int32_t score_stride, const dsa_seqs* seqs,
                           int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                           int32_t* pool_ids, int32_t* indices, void* workspace, size_t workspace_bytes,
                           void* stream) {
    int st = groups_common(dims, seqs, num_seqs, T, score_stride, workspace, workspace_bytes);
    if (st || T == 0 || score_stride == 0) return st;
    if (!scores || !q_seq || !q_pos || !indices) return DSA_ERR_NULL;
    return hip_status(dsa_host::launch_topk_groups(*dims, scores, score_stride, *seqs, q_seq, q_pos, T, pool_ids,
                                                   indices, workspace, as_stream(stream)));
}

int dsa_index_scores_select(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                            const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                            int32_t T, int32_t score_stride, float* scores, int32_t* pool_ids, int32_t* indices,
                            void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, true, false, true);
    if (st) return st;
    if (dims->kpool != 4 || !dsa_host::topk_supported(*dims, score_stride)) return DSA_ERR_UNSUPPORTED;
    if (T == 0 || score_stride == 0) return DSA_OK;
    if (T > 65535) return DSA_ERR_SIZE;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !scores || !indices) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    const size_t need = dsa_index_scores_select_workspace_bytes(dims, T, score_stride);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    }
    hipStream_t s = as_stream(stream);
    if (dsa_host::scores_select_grouped(*dims, T, score_stride)) {
        hipError_t e = dsa_host::launch_scores_with_groups(*dims, q_idx, w, pools, *seqs, num_seqs, q_seq, q_pos, T,
                                                           score_stride, scores, workspace, s);
        if (e != hipSuccess) return DSA_ERR_HIP;
        return hip_status(dsa_host::launch_topk_groups(*dims, scores, score_stride, *seqs, q_seq, q_pos, T,
                                                       pool_ids, indices, workspace, s));
    }
    hipError_t e = dsa_host::launch_index_scores(*dims, q_idx, w, pools, *seqs, num_seqs, q_seq, q_pos, T, score_stride,
                                                 scores, s);
    if (e != hipSuccess) return DSA_ERR_HIP;
    return hip_status(dsa_host::launch_topk(*dims, scores, score_stride, *seqs, q_seq, q_pos, T, pool_ids,
                                            indices, workspace, s));
}

static size_t chunk_scores_bytes(int32_t chunk, int32_t score_stride) {
    return ((size_t)chunk * (size_t)score_stride * 4 + 255) / 256 * 256;
}

// The chunked selection selects each row in one pass when rows have at most
// 40,960 pools; else it keeps 64-pool group lists in the scoring pass (then
// selects from them) when the geometry allows it, else sorts score tiles.
static bool chunked_grouped(const dsa_dims* d, int32_t chunk, int32_t score_stride) {
    return !dsa_host::topk_direct(score_stride) &&
           dsa_host::scores_lists_short(*d, std::min<int32_t>(chunk, 64), score_stride);
}

size_t dsa_index_select_chunked_workspace_bytes(const dsa_dims* dims, int32_t chunk, int32_t score_stride) {
    if (check_dims(dims) != DSA_OK || chunk <= 0 || score_stride <= 0) return 0;
    if (chunked_grouped(dims, chunk, score_stride))
        return chunk_scores_bytes(chunk, score_stride) + dsa_host::scores_select_group_bytes(chunk);
    return chunk_scores_bytes(chunk, score_stride) + dsa_host::topk_workspace_bytes(*dims, chunk, score_stride);
}

int dsa_index_select_chunked(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                             const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                             int32_t T, int32_t score_stride, int32_t chunk, int32_t* pool_ids, int32_t* indices,
                             void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0 || score_stride < 0 || chunk <= 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, true, false, true);
    if (st) return st;
    if (dims->kpool != 4 || !dsa_host::topk_supported(*dims, score_stride)) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if (score_stride == 0) return DSA_ERR_SIZE;
    if (chunk > 65535) return DSA_ERR_SIZE;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !indices) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(pools, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    const size_t need = dsa_index_select_chunked_workspace_bytes(dims, chunk, score_stride);
    if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    float* scores = reinterpret_cast<float*>(workspace);
    void* tws = reinterpret_cast<char*>(workspace) + chunk_scores_bytes(chunk, score_stride);
    const int HI = dims->idx_heads, DI = dims->idx_dim, K = dims->index_topk / dims->kpool, W = dims->out_width;
    const bool grouped = chunked_grouped(dims, chunk, score_stride);
    hipStream_t s = as_stream(stream);
    for (int32_t t0 = 0; t0 < T; t0 += chunk) {
        const int32_t n = std::min(chunk, T - t0);
        const uint16_t* qi = q_idx + (int64_t)t0 * HI * DI;
        const float* wt = w + (int64_t)t0 * HI;
        int32_t* pid = pool_ids ? pool_ids + (int64_t)t0 * K : nullptr;
        int32_t* idx = indices + (int64_t)t0 * W;
        hipError_t e;
        if (grouped) {
            e = dsa_host::launch_scores_lists(*dims, qi, wt, pools, *seqs, num_seqs, q_seq + t0, q_pos + t0, n,
                                              score_stride, scores, tws, s);
            if (e != hipSuccess) return DSA_ERR_HIP;
            e = dsa_host::launch_topk_groups(*dims, scores, score_stride, *seqs, q_seq + t0, q_pos + t0, n, pid, idx,
                                             tws, s);
        } else {
            e = dsa_host::launch_index_scores(*dims, qi, wt, pools, *seqs, num_seqs, q_seq + t0, q_pos + t0, n,
                                              score_stride, scores, s);
            if (e != hipSuccess) return DSA_ERR_HIP;
            e = dsa_host::launch_topk(*dims, scores, score_stride, *seqs, q_seq + t0, q_pos + t0, n, pid, idx, tws, s);
        }
        if (e != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

int dsa_expand_selection(const dsa_dims* dims, const int32_t* pool_ids, const dsa_seqs* seqs,
                         int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T,
                         int32_t* indices, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (T < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, true, false, false);
    if (st) return st;
    if (T == 0) return DSA_OK;
    if (!pool_ids || !q_seq || !q_pos || !indices) return DSA_ERR_NULL;
    return hip_status(dsa_host::launch_expand(*dims, pool_ids, *seqs, q_seq, q_pos, T, indices,
                                              as_stream(stream)));
}

size_t dsa_sparse_mla_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t num_splits) {
    if (check_dims(dims) != DSA_OK || T <= 0 || num_splits < 0) return 0;
    return dsa_host::plan_sparse_mla(*dims, T, num_splits, DSA_BF16).ws_bytes;
}

int dsa_sparse_mla(const dsa_dims* dims, const void* q, int q_dtype, const int8_t* cache,
                   int64_t cache_rows, const int32_t* indices, int32_t T, float scale, void* out,
                   int out_dtype, float* lse, int32_t num_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (T < 0 || cache_rows < 0 || num_splits < 0) return DSA_ERR_SIZE;
    if (dims->latent_dim % 64 != 0 || dims->latent_dim > 1024) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if (T > 65535) return DSA_ERR_SIZE;
    if (!q || !cache || !indices || !out) return DSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16)) return DSA_ERR_ALIGN;
    const dsa_host::MlaPlan plan = dsa_host::plan_sparse_mla(*dims, T, num_splits, q_dtype);
    if (plan.ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan.ws_bytes) return DSA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    }
    return hip_status(dsa_host::launch_sparse_mla(*dims, plan, q, q_dtype, cache, indices, T, scale, out,
                                                  out_dtype, lse, workspace, as_stream(stream)));
}

size_t dsa_sparse_mla_noalloc_scratch_bytes(void) { return dsa::kNoAllocScratchBytes; }

int dsa_sparse_mla_noalloc(const dsa_dims* dims, const void* q, int q_dtype, const int8_t* cache,
                           int64_t cache_rows, const int32_t* indices, int32_t T, float scale, void* out,
                           int out_dtype, float* lse, int32_t num_splits, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (T < 0 || cache_rows < 0 || num_splits < 0) return DSA_ERR_SIZE;
    if (dims->latent_dim % 64 != 0 || dims->latent_dim > 1024) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if (T > 65535) return DSA_ERR_SIZE;
    if (!q || !cache || !indices || !out) return DSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16)) return DSA_ERR_ALIGN;
    const dsa_host::MlaPlan plan = dsa_host::plan_sparse_mla(*dims, T, num_splits, q_dtype);
    if (plan.ws_bytes > dsa::kNoAllocScratchBytes) return DSA_ERR_SCRATCH;
    void* ws = nullptr;
    if (plan.ws_bytes > 0) {
        st = hip_status(dsa_host::noalloc_scratch(&ws));
        if (st) return st;
    }
    return hip_status(dsa_host::launch_sparse_mla(*dims, plan, q, q_dtype, cache, indices, T, scale, out,
                                                  out_dtype, lse, ws, as_stream(stream)));
}

int dsa_topk_sparse_mla(const dsa_dims* dims, const float* scores, int32_t score_stride, const dsa_seqs* seqs,
                        int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* pool_ids,
                        int32_t* indices, const void* select_workspace, size_t select_workspace_bytes,
                        const void* q, int q_dtype, const int8_t* cache, int64_t cache_rows, float scale, void* out,
                        int out_dtype, float* lse, int32_t num_splits, void* mla_workspace,
                        size_t mla_workspace_bytes, void* stream) {
    // the selection half: what dsa_topk_select_groups checks
    int st = groups_common(dims, seqs, num_seqs, T, score_stride, const_cast<void*>(select_workspace),
                           select_workspace_bytes);
    if (st) return st;
    if (T == 0) return DSA_OK;
    if (score_stride == 0) return DSA_ERR_UNSUPPORTED;
    if (!scores || !q_seq || !q_pos || !indices) return DSA_ERR_NULL;
    // the attention half: what dsa_sparse_mla checks
    if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (cache_rows < 0 || num_splits < 0) return DSA_ERR_SIZE;
    if (dims->latent_dim % 64 != 0 || dims->latent_dim > 1024) return DSA_ERR_UNSUPPORTED;
    if (!q || !cache || !out) return DSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16)) return DSA_ERR_ALIGN;
    const dsa_host::MlaPlan plan = dsa_host::plan_sparse_mla(*dims, T, num_splits, q_dtype);
    if (plan.ws_bytes > 0) {
        if (!mla_workspace || mla_workspace_bytes < plan.ws_bytes) return DSA_ERR_WORKSPACE;
        if (!aligned(mla_workspace, 256)) return DSA_ERR_ALIGN;
    }
    return hip_status(dsa_host::launch_select_mla(*dims, plan, scores, score_stride, *seqs, q_seq, q_pos, T,
                                                  pool_ids, indices, select_workspace, q, q_dtype, cache, scale,
                                                  out, out_dtype, lse, mla_workspace, as_stream(stream)));
}

size_t dsa_decode_step_workspace_bytes(const dsa_dims* dims, int32_t T, int32_t score_stride) {
    if (check_dims(dims) != DSA_OK || T <= 0 || score_stride <= 0) return 0;
    if (!dsa_host::decode_step_supported(*dims, T, score_stride)) return 0;
    return dsa_host::decode_step_workspace_bytes(*dims, T, score_stride);
}

int dsa_decode_step(const dsa_dims* dims, const uint16_t* q_idx, const float* w, const uint16_t* pools,
                    const dsa_seqs* seqs, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                    int32_t T, int32_t score_stride, const void* q, int q_dtype, const int8_t* cache,
                    int64_t cache_rows, float scale, void* out, int out_dtype, float* lse,
                    int32_t* pool_ids, int32_t* indices, void* workspace, size_t workspace_bytes,
                    void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (T < 0 || score_stride < 0 || cache_rows < 0) return DSA_ERR_SIZE;
    st = check_seqs(seqs, num_seqs, true, false, true);
    if (st) return st;
    if (T == 0) return DSA_OK;
    if (q_dtype != DSA_BF16 || !dsa_host::decode_step_supported(*dims, T, score_stride))
        return DSA_ERR_UNSUPPORTED;
    if (!q_idx || !w || !pools || !q_seq || !q_pos || !q || !cache || !out) return DSA_ERR_NULL;
    if (!aligned(q_idx, 16) || !aligned(w, 16) || !aligned(pools, 16) || !aligned(q, 16) ||
        !aligned(cache, 16) || !aligned(out, 16))
        return DSA_ERR_ALIGN;
    const size_t need = dsa_host::decode_step_workspace_bytes(*dims, T, score_stride);
    if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DSA_ERR_ALIGN;
    return hip_status(dsa_host::launch_decode_step(*dims, q_idx, w, pools, *seqs, q_seq, q_pos, T, score_stride,
                                                   reinterpret_cast<const uint16_t*>(q), cache, scale, out,
                                                   out_dtype, lse, pool_ids, indices, workspace,
                                                   as_stream(stream)));
}

int dsa_decode_step_status(const void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return DSA_ERR_NULL;
    if (workspace_bytes < 12) return DSA_ERR_WORKSPACE;
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, reinterpret_cast<const char*>(workspace) + 8, 4, hipMemcpyDeviceToHost,
                                  as_stream(stream));
    if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
    if (e != hipSuccess) return DSA_ERR_HIP;
    return word ? DSA_ERR_TIMEOUT : DSA_OK;
}

}  // extern "C"
