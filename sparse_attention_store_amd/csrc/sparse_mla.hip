// sparse_mla: NoPE MLA over the rows an index list selects from the INT8
// latent cache, with the dequantisation fused in ([Kernels] Included and
// Install: one shared 512-d K/V latent, split-KV decode, bf16 products with
// fp32 accumulation and softmax, negative indices as padding; [Ref]
// Functions: mla_masked_attention).
//
// Both MFMA kernels convert the INT8 codes exactly to bf16 (|code| <= 127),
// keep the row scale and the softmax scale out of the products (applied to S
// in fp32), run an online softmax in the exp2 domain, and feed P' = p * scale
// to the PV product split into bf16 hi + lo parts (two MFMAs sharing the V
// operand): the weights then carry ~16 significant bits, which a single
// dominant row of a heavy-tailed latent (|o| ~ 100) needs to stay within
// 2e-2 absolute.
//
// k_mla_rows<RT, NW> (16 heads per workgroup; decode).  The list is walked
// in chunks of 16 RT NW rows (here RT = 1, NW = 8: 128-row chunks, one
// 512-thread workgroup per CU, two waves per SIMD to hide each other's
// latencies); each of the NW waves owns RT 16-row tiles of a chunk:
//  * q (16 heads x 512) is read once per workgroup, before the dependent
//    chain index -> rows, and handed to the waves through LDS (every wave
//    needs all of it: 4 copies per workgroup from L2 cost more than the
//    row gather itself);
//  * the 4 lanes that share a row read it straight into the K operand of
//    S^T = K Q^T (v_mfma_f32_16x16x32_bf16, rows = M, heads = N), 64
//    contiguous bytes per load instruction (lane group g takes bytes
//    64 i + 16 g .. +16); the reduction axis is permuted identically in K and
//    Q, so q is loaded to match and no LDS pass is needed for S;
//  * during the conversion each wave also writes its rows to LDS as bf16
//    (code + 128); the per-head chunk max is exchanged through LDS, and
//    P' = p * row scale goes to LDS as bf16 hi + lo, [head][row];
//  * O^T += V^T P'^T is split by columns: each wave accumulates its own
//    512 / NW columns over every row of the chunk (8-byte LDS reads of 4 adjacent
//    columns assembled with v_perm).  Rows are placed with bits 2 and 3 of
//    the slot swapped so that both the 16-byte writes and the 8-byte reads
//    are free of bank conflicts;
//  * the running max is only raised when a chunk exceeds it by more than
//    2^8, so the accumulators are rescaled rarely (never in a one-chunk
//    split); at the end the waves add up l and the P' sums through LDS.
//
// k_mla_mfma<HT> (16*HT heads per workgroup, HT = 2 or 4; prefill and
// many-query batches).  The workgroup walks 64-row chunks staged in LDS as
// bf16, a wave gathering whole rows (lanes over a row's codes, so its 16-byte
// LDS stores are consecutive).  For S and the softmax the waves own head
// tiles (waves sharing a tile split the rows and exchange their partial max
// and sum); for P'V they own column groups of every head tile, so each V
// operand is read from LDS once, with the per-head rescale and final sums
// handed over through LDS.
//
// One split writes the normalised output directly; several splits write
// (m, l, unnormalised O) partials that k_mla_combine merges in split order,
// so results are deterministic for a given split count.  Empty chunks are
// skipped; an empty split contributes (m = -inf, l = 0) and is ignored.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "mla_core.h"

namespace dsa {

template <int RT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_mla_rows(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int row_bytes,
    const int32_t* __restrict__ indices, int W, int H, float scale_log2, int chunks_per_split,
    int splits, float* __restrict__ part_o, MlaPartial* __restrict__ part_ml,
    void* __restrict__ out, int out_f32, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) MlaRowsSmemT<RT, NW> sm;
    constexpr int CH = 16 * RT * NW;
    const int split = blockIdx.x, t = blockIdx.z;
    const int nchunks = (W + CH - 1) / CH;
    const int c_begin = split * chunks_per_split;
    const int c_end = min(c_begin + chunks_per_split, nchunks);
    const int32_t* irow = indices + (int64_t)t * W;
    const int head0 = blockIdx.y * 16;
    mla_rows_split<RT, false, NW>(sm, [&](int i) { return mla_q_piece<64 * NW>(q, t, H, head0, i); }, cache, row_bytes,
                                  [&](int pos) { return irow[pos]; }, W, H, scale_log2, t, head0, split, c_begin,
                                  c_end, splits, part_o, part_ml, out, out_f32, lse);
}

// ------------------------------------------------------------------ k_mla_mfma
template <int HT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_mla_mfma(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int row_bytes,
    const int32_t* __restrict__ indices, int W, int H, float scale_log2, int chunks_per_split,
    int splits, float* __restrict__ part_o, MlaPartial* __restrict__ part_ml,
    void* __restrict__ out, int out_f32, float* __restrict__ lse) {
    constexpr int NT = 64 * NW;
    constexpr int HPW = 16 * HT;
    constexpr int WPHT = NW / HT;         // waves per head tile
    constexpr int RPW = 4 / WPHT;         // 16-row tiles per wave (S)
    constexpr int NGP = 8 / NW;           // 64-column groups per wave (PV, all HT head tiles)
    constexpr int RW = kChunk / NW;       // gathered rows per wave
    static_assert(WPHT * HT == NW && RPW * WPHT == 4 && NGP * NW == 8 && RW * NW == kChunk && RW <= 64,
                  "64-row chunks, 16-row tiles, 64-column groups");
    // The rows of two chunks (the one computed, the next being converted), so
    // that converting chunk c + 1 needs no barrier after chunk c's P'V.
    __shared__ __attribute__((aligned(16))) uint16_t kv[2][kChunk * kKVRow];
    __shared__ __attribute__((aligned(16))) uint16_t pl[2][HPW * kPRow];   // P' hi, lo
    __shared__ float rs[kChunk];
    __shared__ int rvalid[kChunk];
    __shared__ float red_max[NW][16];
    __shared__ float red_sum[NW][16];
    __shared__ __attribute__((aligned(16))) float alpha_lds[HPW];   // per head: the chunk's rescale of O
    __shared__ __attribute__((aligned(16))) float lsum_lds[HPW];    // per head: the final softmax sum
    __shared__ int chunk_any[2][NW];
    __shared__ int idx_lds[kMaxSplitRows];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, hg = blockIdx.y, t = blockIdx.z;
    const int ht = wave / WPHT, sub = wave % WPHT;
    const int head0 = hg * HPW + ht * 16;
    const int n16 = lane & 15, g4 = lane >> 4;

    // Q (A operand of S): head head0 + n16, k = j*32 + g4*8 + e.
    u32x4 qa[16];
    {
        const uint16_t* qr = q + ((int64_t)t * H + head0 + n16) * kD + g4 * 8;
#pragma unroll
        for (int j = 0; j < 16; ++j) qa[j] = *reinterpret_cast<const u32x4*>(qr + j * 32);
    }

    float m_run[4], l_run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
    // O: column groups NGP w .. NGP w + NGP - 1 of every head tile; lane holds
    // heads 16 ht' + 4 g4 + i, columns 64 grp + 4 n16 + tt
    f32x4 oacc[NGP][HT][4];
#pragma unroll
    for (int gi = 0; gi < NGP; ++gi)
#pragma unroll
        for (int h = 0; h < HT; ++h)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) oacc[gi][h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (W + kChunk - 1) / kChunk;
    const int c_begin = split * chunks_per_split;
    const int c_end = min(c_begin + chunks_per_split, nchunks);
    const int32_t* idx_row = indices + (int64_t)t * W;

    // Row gather: wave w takes the chunk's rows RW w .. RW w + RW - 1, lane l
    // the 8 codes 8 l .. 8 l + 7 of each (one 8-byte load a row: 512
    // contiguous bytes a wave).  Its bf16 stores to LDS are then 16
    // consecutive bytes a lane, so the 8 lanes of a store phase fill 128
    // consecutive bytes, one per bank; lanes that each held a 64-code segment
    // of one row stored 128 bytes apart, all 8 into the same 4 banks.  The
    // split's slice of the index list is staged in LDS once, so the loop
    // issues the rows of chunk c+2 before chunk c computes without any
    // dependent global load in between.
    const int split_rows = (c_end - c_begin) * kChunk;
    for (int i = tid; i < split_rows; i += NT) {
        const int pos = c_begin * kChunk + i;
        idx_lds[i] = pos < W ? idx_row[pos] : -1;
    }
    lds_barrier();
    u32x2 raw[RW];
    float rsc = 0.f;                                 // lane k < RW: the scale of the wave's row k
    // lane k < RW: the id of the wave's row k in chunk c (-1: empty slot)
    auto row_ids = [&](int c) { return idx_lds[(c - c_begin) * kChunk + RW * wave + min(lane, RW - 1)]; };
    auto load_rows = [&](int c) {
        const int mine = row_ids(c);
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            const int idx = __builtin_amdgcn_readlane(mine, k);
            // an empty slot reads through an empty range: zeros
            const __amdgpu_buffer_rsrc_t rr =
                buffer_rsrc(cache + (int64_t)max(idx, 0) * row_bytes, idx >= 0 ? (uint32_t)kD : 0u);
            raw[k] = __builtin_amdgcn_raw_buffer_load_b64(rr, (uint32_t)lane * 8u, 0, 0);
        }
        rsc = (lane < RW && mine >= 0) ? *reinterpret_cast<const float*>(cache + (int64_t)mine * row_bytes + kD) : 0.f;
    };
    // Chunk c's rows to bf16 in kv[buf], its row scales and validity, then
    // the request for chunk c + 2's rows.  The writes are safe without a
    // barrier of their own: kv[buf] was last read by chunk c - 2's P'V, and
    // rs / rvalid by chunk c - 1's softmax, both before chunk c - 1's last
    // barrier; chunk_any alternates too, as a wave may write chunk c's while
    // another still reads chunk c - 1's.
    auto convert = [&](int c, int buf) {
        const int mine = row_ids(c);
        if (lane < RW) { rs[RW * wave + lane] = rsc; rvalid[RW * wave + lane] = mine >= 0; }
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            uint32_t b0, b1, b2, b3;
            int8x4_to_bf16x4(raw[k][0], b0, b1);
            int8x4_to_bf16x4(raw[k][1], b2, b3);
            *reinterpret_cast<u32x4*>(&kv[buf][(RW * wave + k) * kKVRow + 8 * lane]) = u32x4{b0, b1, b2, b3};
        }
        if (c + 1 < c_end) load_rows(c + 1);
        const unsigned long long vote = __ballot(lane < RW && mine >= 0);
        if (lane == 0) chunk_any[buf][wave] = vote != 0ull;
    };
    if (c_begin < c_end) {
        load_rows(c_begin);
        convert(c_begin, 0);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1;
        const uint16_t* kvb = kv[buf];
        lds_barrier();                                   // chunk c converted; chunk c - 1's P'V done
        int any = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) any |= chunk_any[buf][i];
        if (!any) {                                      // empty chunk
            if (c + 1 < c_end) convert(c + 1, buf ^ 1);
            continue;
        }

        // ---- 2. S for this wave's head tile and row tiles sub*RPW .. sub*RPW+RPW-1
        f32x4 sacc[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int rt = sub * RPW + rr;
            const uint16_t* kr = &kvb[(rt * 16 + n16) * kKVRow + g4 * 8];
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 16; ++j)
                a = mfma16(as_bf16x8(qa[j]), as_bf16x8(*reinterpret_cast<const u32x4*>(kr + j * 32)), a);
            sacc[rr] = a;
        }
        // ---- 3. online softmax (log2 domain); lane holds row rt*16+n16, heads 4*g4+i
        float z[RPW][4];
        float cmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int row = (sub * RPW + rr) * 16 + n16;
            const bool ok = rvalid[row] != 0;
            const float sc = rs[row] * scale_log2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[rr][i] = ok ? sacc[rr][i] * sc : -INFINITY;
                cmax[i] = fmaxf(cmax[i], z[rr][i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cmax[i] = row16_max(cmax[i]);
        if (n16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red_max[wave][4 * g4 + i] = cmax[i];
        lds_barrier();
        float m_new[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mc = red_max[ht * WPHT][4 * g4 + i];
#pragma unroll
            for (int s2 = 1; s2 < WPHT; ++s2) mc = fmaxf(mc, red_max[ht * WPHT + s2][4 * g4 + i]);
            m_new[i] = fmaxf(m_run[i], mc);
        }
        // the rescale of O for this tile's heads, published for the P'V waves
        // (read after the next barrier; rewritten only after the next chunk's
        // first two barriers, when every wave is done with it)
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) alpha[i] = m_run[i] == -INFINITY ? 0.f : exp2f(m_run[i] - m_new[i]);
        if (sub == 0 && n16 == 0)
            *reinterpret_cast<f32x4*>(&alpha_lds[ht * 16 + 4 * g4]) = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
        float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int row = (sub * RPW + rr) * 16 + n16;
            const float rsv = rs[row];
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = m_new[i] == -INFINITY ? 0.f : exp2f(z[rr][i] - m_new[i]);
                psum[i] += p;
                x[i] = p * rsv;
            }
            // Lanes 2k and 2k + 1 (rows 2k, 2k + 1) swap one pair of heads
            // each, so that lane 2k + e holds heads 2e, 2e + 1 of both rows
            // and stores them as two 4-byte words (two rows of one head).
            uint32_t hp[2], lp[2];
            split_bf16x2(x[0], x[1], hp[0], lp[0]);
            split_bf16x2(x[2], x[3], hp[1], lp[1]);
            const int e = n16 & 1;
            const int o = (ht * 16 + 4 * g4 + 2 * e) * kPRow + (row & ~1);
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
                const uint32_t* v = hl ? lp : hp;
                const uint32_t mine = e ? v[1] : v[0];
                const uint32_t other = dpp_u32<0xB1, 0xF>(e ? v[0] : v[1], 0u);   // quad_perm [1,0,3,2]
                const uint32_t r_even = e ? other : mine, r_odd = e ? mine : other;
                *reinterpret_cast<uint32_t*>(&pl[hl][o]) = __builtin_amdgcn_perm(r_odd, r_even, 0x05040100u);
                *reinterpret_cast<uint32_t*>(&pl[hl][o + kPRow]) = __builtin_amdgcn_perm(r_odd, r_even, 0x07060302u);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) psum[i] = row16_sum(psum[i]);
        if (n16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red_sum[wave][4 * g4 + i] = psum[i];
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ls = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < WPHT; ++s2) ls += red_sum[ht * WPHT + s2][4 * g4 + i];
            l_run[i] = l_run[i] * alpha[i] + ls;
            m_run[i] = m_new[i];
        }

        // ---- 4. O += P' V over this wave's column groups and every head
        //      tile: each V operand is read once and used HT times
#pragma unroll
        for (int h = 0; h < HT; ++h) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(&alpha_lds[16 * h + 4 * g4]);
#pragma unroll
            for (int gi = 0; gi < NGP; ++gi)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) oacc[gi][h][tt] *= al;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int row0 = ks * 32 + g4 * 8;
#pragma unroll
            for (int gi = 0; gi < NGP; ++gi) {
                const int col0 = 64 * (NGP * wave + gi) + 4 * n16;
                u32x2 v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const u32x2*>(&kvb[(row0 + e) * kKVRow + col0]);
                u32x4 bb[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int wd = tt >> 1;
                    const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;
                    bb[tt][0] = __builtin_amdgcn_perm(v[1][wd], v[0][wd], sel);
                    bb[tt][1] = __builtin_amdgcn_perm(v[3][wd], v[2][wd], sel);
                    bb[tt][2] = __builtin_amdgcn_perm(v[5][wd], v[4][wd], sel);
                    bb[tt][3] = __builtin_amdgcn_perm(v[7][wd], v[6][wd], sel);
                }
#pragma unroll
                for (int h = 0; h < HT; ++h) {
                    const int po = (h * 16 + n16) * kPRow + ks * 32 + g4 * 8;
                    const bf16x8 a_hi = as_bf16x8(*reinterpret_cast<const u32x4*>(&pl[0][po]));
                    const bf16x8 a_lo = as_bf16x8(*reinterpret_cast<const u32x4*>(&pl[1][po]));
                    // the four hi products, then the four lo ones: no MFMA waits
                    // on the one just issued
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) oacc[gi][h][tt] = mfma16(a_hi, as_bf16x8(bb[tt]), oacc[gi][h][tt]);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) oacc[gi][h][tt] = mfma16(a_lo, as_bf16x8(bb[tt]), oacc[gi][h][tt]);
                }
            }
        }
        if (c + 1 < c_end) convert(c + 1, buf ^ 1);
    }

    // ---- epilogue.  The softmax totals are the head tiles' (lanes n16 = 0 of
    // their first wave); the output is written by the P'V waves: lane holds
    // heads 16 h + 4 g4 + i, columns 64 grp + 4 n16 + tt.
    if (sub == 0 && n16 == 0) {
        *reinterpret_cast<f32x4*>(&lsum_lds[ht * 16 + 4 * g4]) = f32x4{l_run[0], l_run[1], l_run[2], l_run[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = head0 + 4 * g4 + i;
            if (splits == 1) {
                if (lse)
                    lse[(int64_t)t * H + head] = l_run[i] > 0.f ? (m_run[i] + log2f(l_run[i])) * kLn2 : -INFINITY;
            } else {
                part_ml[((int64_t)t * splits + split) * H + head] = MlaPartial{m_run[i], l_run[i]};
            }
        }
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&lsum_lds[16 * h + 4 * g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = hg * HPW + 16 * h + 4 * g4 + i;
            if (splits == 1) {
                const float inv = lv[i] > 0.f ? 1.0f / lv[i] : 0.f;
                const int64_t orow = ((int64_t)t * H + head) * kD;
#pragma unroll
                for (int gi = 0; gi < NGP; ++gi) {
                    const int col = 64 * (NGP * wave + gi) + 4 * n16;
                    f32x4 v = {oacc[gi][h][0][i] * inv, oacc[gi][h][1][i] * inv, oacc[gi][h][2][i] * inv,
                               oacc[gi][h][3][i] * inv};
                    if (out_f32) {
                        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow + col) = v;
                    } else {
                        u32x2 pk;
                        pk[0] = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
                        pk[1] = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
                        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + orow + col) = pk;
                    }
                }
            } else if (lv[i] > 0.f) {
                float* po = part_o + (((int64_t)t * splits + split) * H + head) * kD;
#pragma unroll
                for (int gi = 0; gi < NGP; ++gi) {
                    const int col = 64 * (NGP * wave + gi) + 4 * n16;
                    *reinterpret_cast<f32x4*>(po + col) =
                        f32x4{oacc[gi][h][0][i], oacc[gi][h][1][i], oacc[gi][h][2][i], oacc[gi][h][3][i]};
                }
            }
        }
    }
}

// Merge split partials in split order: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Every thread issues the loads of its 4 columns of the first kPre splits
// together with the (m, l) loads (one round trip, not two: an empty split's
// partial was never written, so it is dropped by a select, never multiplied);
// the partials are accumulated in split order.  One wave per workgroup and
// 256 columns per wave (blockIdx.z picks the half of the row): the 2 H T
// workgroups spread the loads over more CUs than 128-thread ones would
// (0.35-0.5 us per decode step).
constexpr int kPre = 24;
__global__ __launch_bounds__(64) void k_mla_combine(
    const float* __restrict__ part_o, const MlaPartial* __restrict__ part_ml, int splits, int H,
    void* __restrict__ out, int out_f32, float* __restrict__ lse) {
    const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x + 64 * (int)blockIdx.z, lane = threadIdx.x;
    const float* base = part_o + ((int64_t)t * splits * H + h) * kD + tid * 4;
    const int64_t sstride = (int64_t)H * kD;
    // The first kPre splits' pieces through one bounded buffer descriptor:
    // splits past the last read 0, so the loads need no branch and all leave
    // at once.
    f32x4 pre[kPre];
    {
        const uint32_t rec = (uint32_t)(((int64_t)(splits - 1) * H + 1) * kD * 4);
        const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(part_o + ((int64_t)t * splits * H + h) * kD, rec);
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const u32x4 v = ld_buf128(rp, (uint32_t)(tid * 16 + u * H * kD * 4));
            pre[u] = f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
        }
    }
    // Each wave derives the split weights itself (lane s: split s, at most 64
    // splits), so the two halves of a row need no exchange.
    MlaPartial p = {-INFINITY, 0.f};
    if (lane < splits) p = part_ml[((int64_t)t * splits + lane) * H + h];
    const bool live = p.l > 0.f;
    const float M = wave_allmax(live ? p.m : -INFINITY);
    const float w = live ? exp2f(p.m - M) : 0.f;
    // a fixed tree over lanes 0..63 (every lane the same bits): deterministic
    const float L = wave_allsum(p.l * w);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const float wu = u < splits ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)) : 0.f;
        const f32x4 c = pre[u] * wu;
        if (wu > 0.f) acc += c;
    }
    for (int s = kPre; s < splits; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
        const f32x4 v = *reinterpret_cast<const f32x4*>(base + s * sstride);
        if (ws > 0.f) acc += v * ws;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    acc *= inv;
    const int64_t orow = ((int64_t)t * H + h) * kD + tid * 4;
    if (out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow) = acc;
    } else {
        u32x2 pk;
        pk[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        pk[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + orow) = pk;
    }
    if (lse && tid == 0) lse[(int64_t)t * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// fp32 vector kernel for other shapes (tiny geometry, fp32 q): one wave per
// (query, head), one pass over the list with an online softmax.
template <bool Q_F32>
__global__ __launch_bounds__(64) void k_mla_generic(
    const void* __restrict__ q, const uint8_t* __restrict__ cache, int row_bytes,
    const int32_t* __restrict__ indices, int W, int H, int D, float scale,
    void* __restrict__ out, int out_f32, float* __restrict__ lse) {
    constexpr int MAXV = 16;                         // D <= 1024
    const int h = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
    const int vpl = D / 64;
    float qv[MAXV], o[MAXV];
    const int64_t qoff = ((int64_t)t * H + h) * D + lane * vpl;
#pragma unroll
    for (int e = 0; e < MAXV; ++e) {
        o[e] = 0.f;
        qv[e] = 0.f;
        if (e < vpl)
            qv[e] = Q_F32 ? reinterpret_cast<const float*>(q)[qoff + e]
                          : bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[qoff + e]);
    }
    float m = -INFINITY, l = 0.f;
    const int32_t* ir = indices + (int64_t)t * W;
    for (int j = 0; j < W; ++j) {
        const int idx = ir[j];
        if (idx < 0) continue;
        const int8_t* rowp = reinterpret_cast<const int8_t*>(cache + (int64_t)idx * row_bytes);
        const float s = *reinterpret_cast<const float*>(rowp + D);
        float code[MAXV];
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < MAXV; ++e) {
            code[e] = e < vpl ? (float)rowp[lane * vpl + e] : 0.f;
            dot += qv[e] * code[e];
        }
        dot = wave_sum(dot);
        const float zz = scale * s * dot;
        const float mn = fmaxf(m, zz);
        const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
        const float p = expf(zz - mn);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < MAXV; ++e) o[e] = o[e] * alpha + p * s * code[e];
        m = mn;
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t ooff = ((int64_t)t * H + h) * D + lane * vpl;
#pragma unroll
    for (int e = 0; e < MAXV; ++e) {
        if (e < vpl) {
            if (out_f32) reinterpret_cast<float*>(out)[ooff + e] = o[e] * inv;
            else reinterpret_cast<uint16_t*>(out)[ooff + e] = (uint16_t)f32_to_bf16_rne(o[e] * inv);
        }
    }
    if (lse && lane == 0) lse[(int64_t)t * H + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace dsa

namespace dsa_host {

MlaPlan plan_sparse_mla(const dsa_dims& d, int32_t T, int32_t num_splits, int q_dtype) {
    MlaPlan p{};
    p.mfma = q_dtype == DSA_BF16 && d.latent_dim == dsa::kD && d.mla_heads % 16 == 0;
    if (!p.mfma || T <= 0) {
        p.head_tiles = 1;
        p.head_groups = d.mla_heads;
        p.rows_chunk = dsa::kRChunk;
        p.splits = 1;
        p.chunks_per_split = 1;
        p.ws_bytes = 0;
        return p;
    }
    const int cu = device_info().cu_count;
    const int tiles16 = d.mla_heads / 16;
    int ht = 1;
    if ((int64_t)T * tiles16 >= 2 * cu) ht = tiles16 % 4 == 0 ? 4 : (tiles16 % 2 == 0 ? 2 : 1);
    p.head_tiles = ht;
    p.head_groups = tiles16 / ht;
    // k_mla_rows walks 128-row chunks; k_mla_mfma 64-row chunks with the
    // split's index slice staged in LDS (at most kMaxSplitRows entries).
    p.rows_chunk = dsa::kRChunk;
    const int chunk = ht == 1 ? p.rows_chunk : dsa::kChunk;
    const int nchunks = (int)cdiv(d.out_width, chunk);
    int want;
    if (num_splits > 0) {
        want = num_splits < nchunks ? num_splits : nchunks;
    } else {
        const int64_t base = (int64_t)T * p.head_groups;
        want = base >= cu ? 1 : (int)std::min<int64_t>(nchunks, cdiv(cu, base));
    }
    if (want > dsa::kMaxSplits) want = dsa::kMaxSplits;
    if (ht != 1) {
        const int min_splits = (int)cdiv(nchunks, dsa::kMaxSplitRows / dsa::kChunk);
        if (want < min_splits) want = min_splits;
    }
    p.chunks_per_split = (int)cdiv(nchunks, want);
    p.splits = (int)cdiv(nchunks, p.chunks_per_split);
    p.ws_bytes = p.splits > 1
                     ? (size_t)T * p.splits * d.mla_heads * (dsa::kD * sizeof(float) + sizeof(dsa::MlaPartial))
                     : 0;
    return p;
}

hipError_t launch_sparse_mla(const dsa_dims& d, const MlaPlan& plan, const void* q, int q_dtype,
                             const int8_t* cache, const int32_t* indices, int32_t T, float scale,
                             void* out, int out_dtype, float* lse, void* ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int H = d.mla_heads, W = d.out_width;
    const int out_f32 = out_dtype == DSA_F32;
    const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cache);
    if (!plan.mfma) {
        dim3 grid((unsigned)H, (unsigned)T);
        if (q_dtype == DSA_F32)
            hipLaunchKernelGGL((dsa::k_mla_generic<true>), grid, dim3(64), 0, s, q, c8, d.row_bytes, indices, W, H,
                               d.latent_dim, scale, out, out_f32, lse);
        else
            hipLaunchKernelGGL((dsa::k_mla_generic<false>), grid, dim3(64), 0, s, q, c8, d.row_bytes, indices, W, H,
                               d.latent_dim, scale, out, out_f32, lse);
        return hipGetLastError();
    }
    float* part_o = reinterpret_cast<float*>(ws);
    dsa::MlaPartial* part_ml = nullptr;
    if (plan.splits > 1)
        part_ml = reinterpret_cast<dsa::MlaPartial*>(part_o + (size_t)T * plan.splits * H * dsa::kD);
    dim3 grid((unsigned)plan.splits, (unsigned)plan.head_groups, (unsigned)T);
    const float sl2 = scale * dsa::kLog2e;
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
    switch (plan.head_tiles) {
        case 4:
            hipLaunchKernelGGL((dsa::k_mla_mfma<4, 8>), grid, dim3(512), 0, s, q16, c8, d.row_bytes, indices, W, H, sl2,
                               plan.chunks_per_split, plan.splits, part_o, part_ml, out, out_f32, lse);
            break;
        case 2:
            hipLaunchKernelGGL((dsa::k_mla_mfma<2, 4>), grid, dim3(256), 0, s, q16, c8, d.row_bytes, indices, W, H, sl2,
                               plan.chunks_per_split, plan.splits, part_o, part_ml, out, out_f32, lse);
            break;
        default:
            static_assert(16 * 1 * 8 == dsa::kRChunk, "k_mla_rows<1, 8> walks kRChunk-row chunks");
            hipLaunchKernelGGL((dsa::k_mla_rows<1, 8>), grid, dim3(512), 0, s, q16, c8, d.row_bytes, indices, W, H, sl2,
                               plan.chunks_per_split, plan.splits, part_o, part_ml, out, out_f32, lse);
            break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_mla_merge(d, plan, T, ws, out, out_dtype, lse, s);
}

hipError_t launch_mla_merge(const dsa_dims& d, const MlaPlan& plan, int32_t T, void* ws, void* out, int out_dtype,
                            float* lse, hipStream_t s) {
    if (T == 0 || plan.splits == 1) return hipSuccess;
    const int H = d.mla_heads;
    float* part_o = reinterpret_cast<float*>(ws);
    const dsa::MlaPartial* part_ml =
        reinterpret_cast<const dsa::MlaPartial*>(part_o + (size_t)T * plan.splits * H * dsa::kD);
    hipLaunchKernelGGL(dsa::k_mla_combine, dim3((unsigned)H, (unsigned)T, 2), dim3(64), 0, s, part_o, part_ml,
                       plan.splits, H, out, out_dtype == DSA_F32 ? 1 : 0, lse);
    return hipGetLastError();
}

}  // namespace dsa_host
