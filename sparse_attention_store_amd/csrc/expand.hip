// expand_selection: selected pools -> raw cache rows, then the visible tail,
// then -1 up to out_width; every entry is written ([Ref] Functions:
// expand_selection; Traps: the -1 sentinel and the fully written output).
// One workgroup per query; the list is a pure function of the ids, so each
// thread computes its entries independently (coalesced int32 stores).
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

__global__ __launch_bounds__(256) void k_expand(
    const int32_t* __restrict__ pool_ids, const int32_t* __restrict__ first_valid,
    const int64_t* __restrict__ row_base, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int select_k, int W, int kpool,
    int32_t* __restrict__ indices) {
    __shared__ uint32_t s_k;
    const int t = blockIdx.x, tid = threadIdx.x;
    const int b = q_seq[t];
    const int f = first_valid[b];
    const int qp = q_pos[t];
    const int64_t rb = row_base[b];
    const int32_t* ids = pool_ids + (int64_t)t * select_k;
    if (tid == 0) s_k = 0u;
    __syncthreads();
    uint32_t cnt = 0;
    for (int i = tid; i < select_k; i += 256) cnt += ids[i] >= 0;
    if (cnt) atomicAdd(&s_k, cnt);
    __syncthreads();
    const int K = (int)s_k;                                   // front-packed: ids[0..K) are the selection
    const int n_vis = qp >= f ? (qp - f + 1) / kpool : 0;
    const int tail = qp >= f ? (qp - f + 1) - kpool * n_vis : 0;
    const int nsel = kpool * K;
    int32_t* out = indices + (int64_t)t * W;
    for (int j = tid; j < W; j += 256) {
        int64_t v = -1;
        if (j < nsel) v = rb + f + (int64_t)kpool * ids[j / kpool] + (j % kpool);
        else if (j < nsel + tail) v = rb + f + (int64_t)kpool * n_vis + (j - nsel);
        out[j] = (int32_t)v;
    }
}

}  // namespace dsa

namespace dsa_host {

hipError_t launch_expand(const dsa_dims& d, const int32_t* pool_ids, const dsa_seqs& seqs,
                         const int32_t* q_seq, const int32_t* q_pos, int32_t T, int32_t* indices,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(dsa::k_expand, dim3((unsigned)T), dim3(256), 0, s, pool_ids, seqs.first_valid,
                       seqs.row_base, q_seq, q_pos, d.index_topk / d.kpool, d.out_width, d.kpool,
                       indices);
    return hipGetLastError();
}

}  // namespace dsa_host
