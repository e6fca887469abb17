// Paged caches ([Kernels] Install: the INT8 cache allocated as [n / 256, 256,
// 528], blocks of 256 rows; [Flash] What already exists: metadata.py's slot
// mappings for the latent, the per-token indexer state and the pooled state).
// A sequence's block table maps its i-th block of 256 positions to a physical
// block id; physical block k holds latent cache rows 256 k .. 256 k + 255,
// indexer-state (k, gate) rows 256 k .. 256 k + 255, and pool rows
// 64 k .. 64 k + 63.  Position x of sequence b is row
// 256 * table[b][x / 256] + x % 256 of the first two, and pool p is row
// 64 * table[b][p / 64] + p % 64 of the pools (a sequence with L positions has
// at most L / 4 pools, so its pools never need more blocks than its
// positions).  A 64-pool group of the scoring pass is one pool block.
#pragma once
#include "dsa_common.h"

namespace dsa {

constexpr int kPageRows = 256;   // positions per block
constexpr int kPagePools = 64;   // pools per block

struct PagedMap {
    const int32_t* table;        // [num_seqs, stride] physical block ids
    int32_t stride;              // entries per sequence

    __device__ __forceinline__ int64_t block(int b, int64_t i) const {
        return (int64_t)table[(int64_t)b * stride + i];
    }
    __device__ __forceinline__ int64_t row(int b, int64_t x) const {
        return block(b, x >> 8) * kPageRows + (x & (kPageRows - 1));
    }
    __device__ __forceinline__ int64_t pool_row(int b, int64_t p) const {
        return block(b, p >> 6) * kPagePools + (p & (kPagePools - 1));
    }
};

}  // namespace dsa
