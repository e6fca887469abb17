"""Plain CPU definitions of each step of the DSA path (test infrastructure only).

Short page names are defined in this package's ``__init__``.  Each function
states the passage it follows and the reading taken where the pages are
silent.  Nothing here is blocked, fused or reordered beyond what the stated
definition needs; NumPy primitives (matmul, lexsort, exp) are used as steps.
"""
from __future__ import annotations

import numpy as np

INVALID = -1                       # [Ref] Constants: the invalid-index sentinel
AMAX_FLOOR = np.float32(1e-4)      # [Flash] What is quantized: per-token amax floor (borrowed, reading R13)
QMAX = np.float32(127.0)           # symmetric INT8 range; -128 is never produced

__all__ = [
    "INVALID", "AMAX_FLOOR", "QMAX", "row_bytes_for", "quantize_rows", "pack_rows",
    "store_int8", "dequantize_rows", "layer_norm", "slot_softmax", "pool_states",
    "store_bf16", "visible", "visible_pool_count", "index_scores", "topk_pools", "expand_selection",
    "topk_to_mask", "sparse_mla", "masked_attention", "attention_unquantized",
    "quantize_pools", "dequantize_pools", "index_scores_int8", "int8_accuracy",
]


# ---------------------------------------------------------------------------
# O1  INT8 latent row -- [Kernels] Included: store_int8 turns one 512-value
# latent into a 528-byte row made of 512 INT8 codes, one FP32 scale and 12
# zero bytes.  The rounding rule is not printed; the reading used here is an
# IEEE fp32 division followed by round-half-to-even, symmetric +-127, and the
# amax floored at 1e-4 (the floor the [Flash] page prints for per-token INT8).
# The layout, the floor and the rounding mode are readings (parity unpinned
# beyond the invariants the tests check: dequant error <= scale/2, amax maps to
# +-127, zero padding, constant and zero rows).
# ---------------------------------------------------------------------------

def row_bytes_for(latent_dim: int) -> int:
    """Row size: D int8 codes + 4-byte scale, rounded up to 16 bytes (512 -> 528)."""
    return ((latent_dim + 4 + 15) // 16) * 16


def quantize_rows(x: np.ndarray):
    """Per-row dynamic INT8 quantisation in fp32.

    x: float32 [n, D].  Returns (codes int8 [n, D], scales float32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)                         # float32
    scale = np.maximum(amax, AMAX_FLOOR) / QMAX              # float32 / float32 (IEEE)
    ratio = x / scale[:, None]                               # float32 (IEEE division)
    codes = np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)   # rint: ties to even
    return codes, scale.astype(np.float32)


def pack_rows(codes: np.ndarray, scales: np.ndarray, row_bytes: int) -> np.ndarray:
    """Bytes of each row: codes, then the fp32 scale (little endian), then zeros."""
    n, d = codes.shape
    out = np.zeros((n, row_bytes), dtype=np.uint8)
    out[:, :d] = codes.view(np.uint8)
    out[:, d:d + 4] = scales.astype("<f4").view(np.uint8).reshape(n, 4)
    return out


def store_int8(latent: np.ndarray, slots: np.ndarray, cache: np.ndarray) -> None:
    """Write the INT8 row of latent[i] at cache row slots[i]; negative slots are skipped.

    cache: uint8 [rows, row_bytes], modified in place."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    codes, scales = quantize_rows(np.asarray(latent)[keep])
    cache[slots[keep]] = pack_rows(codes, scales, cache.shape[1])


def dequantize_rows(rows: np.ndarray, latent_dim: int) -> np.ndarray:
    """float64 values int8_code * scale of each stored row (uint8 [n, row_bytes]).

    Pinned against rows assembled byte by byte (two's-complement codes, the
    little-endian scale at bytes D .. D+4, pad bytes ignored) and against the
    s/2 round-trip bound of stored rows."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    codes = rows[:, :latent_dim].view(np.int8).astype(np.float64)
    scales = rows[:, latent_dim:latent_dim + 4].copy().view("<f4").astype(np.float64)
    return codes * scales


# ---------------------------------------------------------------------------
# O2  Pools -- [Ref] Traps and Functions (layer_norm, pool_states):
#   * the indexer key norm is a LayerNorm with mean subtraction and a bias;
#   * the pool softmax runs over the slot axis, separately for every channel;
#   * pools begin at the first valid token;
#   * a pool exists only when all kpool slots are valid (7 tokens -> 1 pool).
# Readings: the softmax is over the raw gate values (the path applies no other
# gating); LayerNorm uses the biased variance and an explicit eps.
# ---------------------------------------------------------------------------

def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis in float64: (x - mean) / sqrt(var + eps) * w + b."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + float(eps)) * np.asarray(w, np.float64) + np.asarray(b, np.float64)


def slot_softmax(gate_slots: np.ndarray) -> np.ndarray:
    """Softmax over axis 1 (the pool-slot axis) of gate values [P, kpool, Di]."""
    g = np.asarray(gate_slots, dtype=np.float64)
    e = np.exp(g - g.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def pool_states(k: np.ndarray, gate: np.ndarray, ln_w, ln_b, eps: float,
                first_valid: int, seq_len: int, kpool: int, return_weights: bool = False):
    """Pools of one sequence.  k, gate: [seq_len, Di] indexed by position.

    Pool p gathers positions first_valid + kpool*p + s for s in [0, kpool) and
    equals sum_s softmax_s(gate)[c] * LayerNorm(k)[c] per channel c."""
    n_valid = max(int(seq_len) - int(first_valid), 0)
    n_pools = n_valid // kpool
    di = k.shape[1]
    if n_pools == 0:
        empty = np.zeros((0, di))
        return (empty, np.zeros((0, kpool, di))) if return_weights else empty
    toks = int(first_valid) + np.arange(n_pools)[:, None] * kpool + np.arange(kpool)[None, :]
    y = layer_norm(np.asarray(k)[toks], ln_w, ln_b, eps)         # [P, kpool, Di]
    a = slot_softmax(np.asarray(gate)[toks])                     # [P, kpool, Di]
    pools = (a * y).sum(axis=1)
    return (pools, a) if return_weights else pools


def store_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Pool states are held in bf16 (bf16 pool states with fp32 accumulation are
    the precision the path is specified at; reading R19), so a pool is
    computed in full precision and then rounded once to the 8-bit-significand
    bf16 grid.  Computed directly from the float64 value (no intermediate
    fp32 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                           # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


# ---------------------------------------------------------------------------
# Visibility -- [Ref] Functions (visible): a query sees keys that are causal
# and not padding.  Reading R6/R8: positions first_valid <= x <= q_pos, the
# query sees itself; pool p is visible when its last slot is visible.
# ---------------------------------------------------------------------------

def visible(q_pos: int, first_valid: int, x) -> np.ndarray:
    x = np.asarray(x)
    return (x >= first_valid) & (x <= q_pos)


def visible_pool_count(q_pos: int, first_valid: int, kpool: int) -> int:
    """Pools whose kpool slots all lie in [first_valid, q_pos]."""
    if q_pos < first_valid:
        return 0
    return (int(q_pos) - int(first_valid) + 1) // kpool


# ---------------------------------------------------------------------------
# O3  Scores -- [Ref] Functions (index_scores): matmul, then ReLU, then a
# head-weighted sum; [Flash] checkpoint table: 32 indexer heads x 128.
# Reading R4: no extra scale factor (any is folded into w by the caller).
# ---------------------------------------------------------------------------

def index_scores(q_idx: np.ndarray, w: np.ndarray, pools: np.ndarray, n_vis: int,
                 stride: int | None = None) -> np.ndarray:
    """score[p] = sum_h w[h] * max(0, q_idx[h] . pool[p]) for p < n_vis, -inf after.

    q_idx: [Hi, Di]; w: [Hi]; pools: [>= n_vis, Di].  Returns float64 [stride]."""
    stride = n_vis if stride is None else stride
    out = np.full(stride, -np.inf)
    if n_vis > 0:
        logits = np.asarray(pools[:n_vis], np.float64) @ np.asarray(q_idx, np.float64).T  # [n_vis, Hi]
        out[:n_vis] = (np.maximum(logits, 0.0) * np.asarray(w, np.float64)[None, :]).sum(axis=1)
    return out


# ---------------------------------------------------------------------------
# O4  Top-k -- [Ref] Functions (topk_pools): up to select_k pools per query;
# [Flash] stream C: index_topk 2048 tokens = 512 pools of 4.  The tie rule is
# not printed ([TF402] Credit mentions one without stating it): reading R9
# takes (score descending, pool id ascending), -0 equal to +0, and emits the
# chosen ids in ascending order (R10), padded with INVALID (tie rule: parity
# unpinned by the pages, pinned only by this reading).
# ---------------------------------------------------------------------------

def topk_pools(scores: np.ndarray, n_vis: int, select_k: int) -> np.ndarray:
    ids = np.full(select_k, INVALID, dtype=np.int32)
    k = min(select_k, n_vis)
    if k <= 0:
        return ids
    s = np.asarray(scores[:n_vis], dtype=np.float64)
    order = np.lexsort((np.arange(n_vis), -s))       # primary: -score, secondary: id
    ids[:k] = np.sort(order[:k])
    return ids


# ---------------------------------------------------------------------------
# O5  Expansion -- [Ref] Functions (expand_selection) and the sentinel trap:
# selected pools become their kpool raw positions, the visible tail is
# appended, INVALID fills the rest, and every one of the out_width entries is
# written.  Index values are cache rows row_base + position (reading R11).
# ---------------------------------------------------------------------------

def expand_selection(pool_ids: np.ndarray, first_valid: int, q_pos: int, row_base: int,
                     kpool: int, out_width: int) -> np.ndarray:
    n_vis = visible_pool_count(q_pos, first_valid, kpool)
    rows = []
    for p in pool_ids:
        if p >= 0:
            rows.extend(int(row_base) + int(first_valid) + kpool * int(p) + s for s in range(kpool))
    if q_pos >= first_valid:
        rows.extend(int(row_base) + x for x in range(int(first_valid) + kpool * n_vis, int(q_pos) + 1))
    if len(rows) > out_width:
        raise ValueError("selection does not fit out_width")
    out = np.full(out_width, INVALID, dtype=np.int32)
    out[:len(rows)] = rows
    return out


def topk_to_mask(indices: np.ndarray, row_base: int, seq_len: int) -> np.ndarray:
    """[Ref] Functions (topk_to_mask): boolean mask over the sequence's positions."""
    mask = np.zeros(seq_len, dtype=bool)
    idx = np.asarray(indices)
    idx = idx[idx >= 0] - int(row_base)
    mask[idx] = True
    return mask


# ---------------------------------------------------------------------------
# O6  Sparse NoPE MLA -- [Kernels] Included / Install: attention of 16 query
# heads over one shared 512-d latent that is both K and V, dequantised from
# the INT8 rows, with negative indices as padding; [Ref] Functions
# (mla_masked_attention).  This is the plain softmax-attention definition that
# a split-KV / online-softmax kernel reaches up to rounding order.
# Reading R7/R17/R18: any negative entry is skipped; no valid entry gives a
# zero output and lse = -inf.
# ---------------------------------------------------------------------------

def sparse_mla(q: np.ndarray, cache: np.ndarray, indices: np.ndarray, scale: float,
               latent_dim: int):
    """q: [H, D]; cache: uint8 [rows, row_bytes]; indices: [W].  Returns (o [H, D], lse [H])."""
    idx = np.asarray(indices, dtype=np.int64)
    idx = idx[idx >= 0]
    h = q.shape[0]
    if idx.size == 0:
        return np.zeros((h, latent_dim)), np.full(h, -np.inf)
    kv = dequantize_rows(cache[idx], latent_dim)                  # [n, D]
    z = float(scale) * (np.asarray(q, np.float64) @ kv.T)         # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ kv) / l, (m + np.log(l))[:, 0]


def masked_attention(q: np.ndarray, keys: np.ndarray, mask: np.ndarray, scale: float):
    """Dense attention over all rows of `keys` (K = V) with -inf outside `mask` (brute force)."""
    z = float(scale) * (np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T)
    z = np.where(mask[None, :], z, -np.inf)
    if not mask.any():
        return np.zeros((q.shape[0], keys.shape[1])), np.full(q.shape[0], -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ np.asarray(keys, np.float64)) / l, (m + np.log(l))[:, 0]


def attention_unquantized(q: np.ndarray, latent_rows: np.ndarray, scale: float) -> np.ndarray:
    """Attention over the source (unquantised) latents, for the INT8 accuracy report."""
    return masked_attention(q, latent_rows, np.ones(latent_rows.shape[0], dtype=bool), scale)[0]


# ---------------------------------------------------------------------------
# O2q / O3q  INT8 pool cache -- [Flash] What is quantized (the indexer state
# cache row): the sibling port keeps its indexer cache as INT8 codes with one
# FP32 scale per row.  Readings: the quantiser is the one of the latent rows
# (O1: amax floored at 1e-4, scale = amax / 127 in IEEE fp32, round half to
# even, symmetric +-127), applied to each pool's fp32 state (the state
# precision the page names), with no bf16 step in between and no Hadamard
# rotation: the query stays in bf16 and is not quantised, so an orthonormal
# rotation of both operands would leave q . pool unchanged (reading R20).
# Scores are O3 on the dequantised pools.
# ---------------------------------------------------------------------------

def quantize_pools(pools: np.ndarray):
    """Pool states (any float dtype) -> (codes int8 [P, Di], scales float32 [P]):
    the fp32 state, quantised per row by the O1 formula."""
    return quantize_rows(np.asarray(pools, dtype=np.float64).astype(np.float32))


def dequantize_pools(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 code * scale per pool row."""
    return np.asarray(codes, np.float64) * np.asarray(scales, np.float64)[:, None]


def index_scores_int8(q_idx: np.ndarray, w: np.ndarray, codes: np.ndarray, scales: np.ndarray, n_vis: int,
                      stride: int | None = None) -> np.ndarray:
    """O3 over INT8 pools: sum_h w[h] * max(0, q_idx[h] . (scale_p * code_p)) for p < n_vis, -inf after."""
    n = min(int(n_vis), codes.shape[0])
    return index_scores(q_idx, w, dequantize_pools(codes[:n], scales[:n]), n_vis, stride)


def int8_accuracy(o_int8: np.ndarray, o_ref: np.ndarray):
    """NMSE and cosine similarity of an attention output against a reference
    output (the accuracy figures [Kernels] Measurements reports for INT8 MLA
    against BF16 latents): NMSE = |o - r|^2 / |r|^2, cosine = o.r / (|o| |r|),
    each over one query's heads and channels."""
    o = np.asarray(o_int8, np.float64).ravel()
    r = np.asarray(o_ref, np.float64).ravel()
    return float(np.sum((o - r) ** 2) / np.sum(r * r)), float(o @ r / (np.linalg.norm(o) * np.linalg.norm(r)))
