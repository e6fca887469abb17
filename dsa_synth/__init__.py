"""Seeded synthetic inputs for the DSA decode/prefill path.

This module is shared by the CPU oracle and by the GPU path's tests and bench.
It holds no arithmetic of the method itself: it only describes workload
shapes (sequence lengths, padding, cache row layout, query positions) and draws
seeded random tensors, rounded to bf16 where the workload says so.  The bf16
values returned here are the ground truth for both sides.

Every tensor is generated in fixed blocks from a counter-based Philox stream
keyed by (seed, tensor id, sequence, block), so any block can be regenerated on
its own without materialising the whole tensor.

Workload shapes follow the pages' workloads: GLM-5.3-Flash indexer geometry
(32 heads x 128, kpool 4, index_topk 2048 -- "GLM-5.3-Flash", checkpoint shape
table) and the INT8 MLA contract (16 query heads, 512-d NoPE latent, 528-byte
rows, 2176 index slots -- "GLM-5.3 Kernels", Included / Install sections).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

ROW_BLOCK = 4096      # positions per generated block (latent, k, gate)
QUERY_BLOCK = 256     # queries per generated block (q, q_idx, w)
POISON = 1000.0       # magnitude written at left-padding positions

_TENSOR_IDS = {
    "latent": 1, "k": 2, "gate": 3, "q_idx": 4, "w": 5, "q": 6,
    "ln_w": 7, "ln_b": 8, "lengths": 9, "queries": 10,
}


@dataclass(frozen=True)
class Dims:
    """Indexer + MLA geometry.  Every field is explicit (no defaults)."""
    idx_heads: int
    idx_dim: int
    kpool: int
    index_topk: int
    out_width: int
    mla_heads: int
    latent_dim: int
    row_bytes: int
    ln_eps: float

    @property
    def select_k(self) -> int:
        return self.index_topk // self.kpool


def production_dims(mla_heads: int) -> Dims:
    return Dims(idx_heads=32, idx_dim=128, kpool=4, index_topk=2048,
                out_width=2176, mla_heads=mla_heads, latent_dim=512,
                row_bytes=528, ln_eps=1e-5)


TINY_DIMS = Dims(idx_heads=4, idx_dim=32, kpool=4, index_topk=16, out_width=24,
                 mla_heads=2, latent_dim=64, row_bytes=80, ln_eps=1e-5)


@dataclass
class Workload:
    """One batch of sequences plus the queries issued against them.

    Position x of sequence b (0 <= x < seq_len[b]) lives at cache row
    row_base[b] + x and at indexer-state row tok_base[b] + x.  Positions below
    first_valid[b] are left padding.  Pool p of sequence b lives at pool row
    pool_base[b] + p.
    """
    name: str
    seed: int
    dims: Dims
    first_valid: np.ndarray      # int32 [B]
    seq_len: np.ndarray          # int32 [B]
    row_base: np.ndarray         # int64 [B]
    tok_base: np.ndarray         # int64 [B]
    pool_base: np.ndarray        # int64 [B]
    q_seq: np.ndarray            # int32 [T]
    q_pos: np.ndarray            # int32 [T]
    fp32_mla: bool = False       # latent and q in fp32 (tiny config)
    latent_dist: str = "normal"  # "normal" or "t3" (Student-t, nu = 3)
    weight_dist: str = "uniform"  # per-head indexer weights: "uniform" U(0,1) or "normal"
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.first_valid.shape[0])

    @property
    def T(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def scale(self) -> float:
        return float(self.dims.latent_dim) ** -0.5

    @property
    def total_rows(self) -> int:
        return int(np.max(self.row_base + self.seq_len)) if self.B else 0

    @property
    def total_tokens(self) -> int:
        return int(np.max(self.tok_base + self.seq_len)) if self.B else 0

    def n_pools(self, b: int) -> int:
        """Number of complete pools of sequence b (all kpool slots valid)."""
        v = int(self.seq_len[b]) - int(self.first_valid[b])
        return max(v, 0) // self.dims.kpool

    @property
    def total_pools(self) -> int:
        return int(max(int(self.pool_base[b]) + self.n_pools(b) for b in range(self.B))) if self.B else 0

    def n_vis(self, t: int) -> int:
        """Pools visible to query t (workload bookkeeping used to size buffers)."""
        b = int(self.q_seq[t])
        f = int(self.first_valid[b])
        q = int(self.q_pos[t])
        return (q - f + 1) // self.dims.kpool if q >= f else 0

    @property
    def max_n_vis(self) -> int:
        return max((self.n_vis(t) for t in range(self.T)), default=0)

    def subset_queries(self, idx) -> "Workload":
        idx = np.asarray(idx)
        return dataclasses.replace(self, q_seq=self.q_seq[idx].copy(), q_pos=self.q_pos[idx].copy())


# ----------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# counter-based streams
# ----------------------------------------------------------------------------

def _rng(seed: int, tensor: str, b: int, block: int) -> np.random.Generator:
    tid = _TENSOR_IDS[tensor]
    key = np.array([np.uint64(seed) & np.uint64(0xFFFFFFFFFFFFFFFF),
                    np.uint64((tid << 48) | (b << 32) | block)], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _block_rows(seed, tensor, b, x0, x1, width, sampler):
    """Rows [x0, x1) of a per-sequence tensor generated in ROW_BLOCK blocks."""
    out = np.empty((x1 - x0, width), dtype=np.float32)
    if x1 <= x0:
        return out
    for blk in range(x0 // ROW_BLOCK, (x1 - 1) // ROW_BLOCK + 1):
        lo, hi = blk * ROW_BLOCK, (blk + 1) * ROW_BLOCK
        vals = sampler(_rng(seed, tensor, b, blk), (ROW_BLOCK, width))
        a, c = max(lo, x0), min(hi, x1)
        out[a - x0:c - x0] = vals[a - lo:c - lo]
    return out


def _normal(g, shape):
    return g.standard_normal(shape, dtype=np.float32)


def _student_t3(g, shape):
    return g.standard_t(3.0, size=shape).astype(np.float32)


def _uniform01(g, shape):
    return g.random(shape, dtype=np.float32)


def _poison(vals: np.ndarray, x0: int, first_valid: int) -> np.ndarray:
    n_pad = max(0, min(first_valid - x0, vals.shape[0]))
    if n_pad:
        vals[:n_pad] = np.where(vals[:n_pad] >= 0, POISON, -POISON).astype(np.float32)
    return vals


def gen_latent(wl: Workload, b: int, x0: int, x1: int) -> np.ndarray:
    """MLA latent rows for positions [x0, x1) of sequence b, float32 [n, D].

    bf16-exact unless the workload is fp32.  Left padding is poisoned (+-1e3)."""
    samp = _student_t3 if wl.latent_dist == "t3" else _normal
    v = _block_rows(wl.seed, "latent", b, x0, x1, wl.dims.latent_dim, samp)
    v = _poison(v, x0, int(wl.first_valid[b]))
    return v if wl.fp32_mla else bf16_round(v)


def gen_kgate(wl: Workload, b: int, x0: int, x1: int):
    """Indexer key and gate rows for positions [x0, x1) of sequence b (bf16-exact float32)."""
    di = wl.dims.idx_dim
    f = int(wl.first_valid[b])
    k = _poison(_block_rows(wl.seed, "k", b, x0, x1, di, _normal), x0, f)
    g = _poison(_block_rows(wl.seed, "gate", b, x0, x1, di, _normal), x0, f)
    return bf16_round(k), bf16_round(g)


def gen_ln(wl: Workload):
    """Indexer LayerNorm weight and bias, float32 [Di] each (N(0,1))."""
    di = wl.dims.idx_dim
    w = _rng(wl.seed, "ln_w", 0, 0).standard_normal(di, dtype=np.float32)
    bb = _rng(wl.seed, "ln_b", 0, 0).standard_normal(di, dtype=np.float32)
    return w, bb


def _block_queries(seed, tensor, t0, t1, width, sampler):
    out = np.empty((t1 - t0, width), dtype=np.float32)
    if t1 <= t0:
        return out
    for blk in range(t0 // QUERY_BLOCK, (t1 - 1) // QUERY_BLOCK + 1):
        lo, hi = blk * QUERY_BLOCK, (blk + 1) * QUERY_BLOCK
        vals = sampler(_rng(seed, tensor, 0, blk), (QUERY_BLOCK, width))
        a, c = max(lo, t0), min(hi, t1)
        out[a - t0:c - t0] = vals[a - lo:c - lo]
    return out


def gen_qidx(wl: Workload, t0: int, t1: int) -> np.ndarray:
    d = wl.dims
    v = _block_queries(wl.seed, "q_idx", t0, t1, d.idx_heads * d.idx_dim, _normal)
    return bf16_round(v).reshape(t1 - t0, d.idx_heads, d.idx_dim)


def gen_w(wl: Workload, t0: int, t1: int) -> np.ndarray:
    d = wl.dims
    samp = _uniform01 if wl.weight_dist == "uniform" else _normal
    return _block_queries(wl.seed, "w", t0, t1, d.idx_heads, samp)


def gen_q(wl: Workload, t0: int, t1: int) -> np.ndarray:
    d = wl.dims
    v = _block_queries(wl.seed, "q", t0, t1, d.mla_heads * d.latent_dim, _normal)
    v = v if wl.fp32_mla else bf16_round(v)
    return v.reshape(t1 - t0, d.mla_heads, d.latent_dim)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def _mk(name, seed, dims, fv, sl, row_cap, pool_cap, q_seq, q_pos, **kw) -> Workload:
    fv = np.asarray(fv, dtype=np.int32)
    sl = np.asarray(sl, dtype=np.int32)
    B = fv.shape[0]
    rb = np.arange(B, dtype=np.int64) * np.int64(row_cap)
    pb = np.arange(B, dtype=np.int64) * np.int64(pool_cap)
    return Workload(name=name, seed=seed, dims=dims, first_valid=fv, seq_len=sl,
                    row_base=rb, tok_base=rb.copy(), pool_base=pb,
                    q_seq=np.asarray(q_seq, dtype=np.int32),
                    q_pos=np.asarray(q_pos, dtype=np.int32), **kw)


def _all_positions(sl):
    qs, qp = [], []
    for b, n in enumerate(sl):
        qs += [b] * n
        qp += list(range(n))
    return qs, qp


def tiny(seed: int = 0) -> Workload:
    """64 tokens, 5 left-padded; every position issues a query (decode query = 63)."""
    qs, qp = _all_positions([64])
    return _mk("tiny", seed, TINY_DIMS, [5], [64], 64, 16, qs, qp,
               fp32_mla=True, weight_dist="normal",
               note="tiny geometry; fp32 MLA; N(0,1) values")


def tiny_seven(seed: int = 0) -> Workload:
    """Seven valid tokens, no padding: exactly one pool plus a 3-token tail."""
    qs, qp = _all_positions([7])
    return _mk("tiny_seven", seed, TINY_DIMS, [0], [7], 8, 2, qs, qp,
               fp32_mla=True, weight_dist="normal")


def tiny_padded_six(seed: int = 0) -> Workload:
    """Left padding [P, P, A, B, C, D]: pool 0 is [A, B, C, D]."""
    qs, qp = _all_positions([6])
    return _mk("tiny_padded_six", seed, TINY_DIMS, [2], [6], 8, 2, qs, qp,
               fp32_mla=True, weight_dist="normal")


def tiny_batch(seed: int = 7) -> Workload:
    """The three tiny sequences in one ragged batch (exercises per-sequence bases)."""
    sl = [64, 7, 6]
    qs, qp = _all_positions(sl)
    return _mk("tiny_batch", seed, TINY_DIMS, [5, 0, 2], sl, 64, 16, qs, qp,
               fp32_mla=True, weight_dist="normal")


def decode_32k(seed: int = 1) -> Workload:
    """B=1 decode at context 32,768, 16 MLA heads."""
    return _mk("decode_32k", seed, production_dims(16), [0], [32768], 32768, 8192,
               [0], [32767])


def decode_262k_b8(seed: int = 2) -> Workload:
    """B=8 ragged decode: valid length ~ U[8192, 262144 - p], left padding p ~ U{0..3}."""
    g = _rng(seed, "lengths", 0, 0)
    p = g.integers(0, 4, size=8)
    v = np.array([g.integers(8192, 262144 - int(pi) + 1) for pi in p])
    sl = p + v
    return _mk("decode_262k_b8", seed, production_dims(16), p, sl, 262144, 65536,
               np.arange(8), sl - 1, note="ragged lengths drawn from the seeded stream")


def decode_262k_b8_full(seed: int = 2) -> Workload:
    """Uniform-max variant: all eight sequences hold 262,144 valid tokens."""
    sl = np.full(8, 262144)
    return _mk("decode_262k_b8_full", seed, production_dims(16), np.zeros(8), sl,
               262144, 65536, np.arange(8), sl - 1)


def prefill_4k_on_131k(seed: int = 3) -> Workload:
    """4,096 causal queries appended to a 131,072-token context (B=1, 64 MLA heads)."""
    n_ctx, n_q = 131072, 4096
    sl = n_ctx + n_q
    return _mk("prefill_4k_on_131k", seed, production_dims(64), [0], [sl], sl, sl // 4,
               np.zeros(n_q), np.arange(n_ctx, sl))


def decode_1m_b4(seed: int = 4) -> Workload:
    """B=4 decode at the 1,048,576 maximum position, 64 heads, Student-t(3) latent."""
    fv = [0, 3, 1, 2]
    v = [1048576, 1048573, 1537, 6]
    sl = [a + b for a, b in zip(fv, v)]
    return _mk("decode_1m_b4", seed, production_dims(64), fv, sl, 1048576, 262144,
               np.arange(4), np.array(sl) - 1, latent_dist="t3")


# --- reduced-size workloads with the production geometry (element-wise parity) ---

def mini_decode(seed: int = 11) -> Workload:
    """Ragged B=4 batch, production geometry, several queries per sequence.

    Includes a query inside the left padding (empty selection), queries in the
    dense regime (fewer visible pools than the budget) and sparse ones."""
    fv = [0, 1, 3, 2]
    v = [4096, 3001, 2050, 517]
    sl = [a + b for a, b in zip(fv, v)]
    qs, qp = [], []
    g = _rng(seed, "queries", 0, 0)
    for b in range(4):
        qs.append(b); qp.append(sl[b] - 1)
        for x in g.integers(fv[b], sl[b], size=3):
            qs.append(b); qp.append(int(x))
    qs.append(2); qp.append(1)          # inside the padding of sequence 2
    qs.append(1); qp.append(2058)       # budget boundary: 514 visible pools
    return _mk("mini_decode", seed, production_dims(16), fv, sl, 4100, 1025, qs, qp)


def mini_decode_64(seed: int = 14) -> Workload:
    """The most queries a decode launch takes: 64, over 8 ragged sequences
    (8 queries each at seeded positions, the last position among them)."""
    fv = [0, 1, 3, 2, 0, 3, 1, 2]
    v = [4096, 3001, 2050, 517, 3900, 2100, 800, 2600]
    sl = [a + b for a, b in zip(fv, v)]
    qs, qp = [], []
    g = _rng(seed, "queries", 0, 0)
    for b in range(8):
        qs.append(b); qp.append(sl[b] - 1)
        for x in g.integers(fv[b], sl[b], size=7):
            qs.append(b); qp.append(int(x))
    return _mk("mini_decode_64", seed, production_dims(16), fv, sl, 4100, 1025, qs, qp)


def mini_prefill(seed: int = 12) -> Workload:
    """Prefill chunk of 200 queries on a 3,000-token context, 64 MLA heads."""
    n_ctx, n_q = 3000, 200
    sl = n_ctx + n_q
    return _mk("mini_prefill", seed, production_dims(64), [0], [sl], sl, sl // 4,
               np.zeros(n_q), np.arange(n_ctx, sl))


def mini_prefill_wide(seed: int = 17) -> Workload:
    """96 causal queries appended to a 180,000-token context (45,024 pools at
    the last query): rows past the single-pass selection's 40,960 pools, so a
    chunked selection keeps 64-pool group lists, 64 heads."""
    n_ctx, n_q = 180000, 96
    sl = n_ctx + n_q
    return _mk("mini_prefill_wide", seed, production_dims(64), [0], [sl], sl, sl // 4,
               np.zeros(n_q), np.arange(n_ctx, sl))


def mini_heavy(seed: int = 13) -> Workload:
    """64 heads, Student-t(3) latent, a mix of sparse, dense and nearly empty lists."""
    fv = [0, 3, 1]
    v = [2500, 777, 6]
    sl = [a + b for a, b in zip(fv, v)]
    return _mk("mini_heavy", seed, production_dims(64), fv, sl, 2504, 626,
               np.arange(3), np.array(sl) - 1, latent_dist="t3")


def mini_long(seed: int = 16) -> Workload:
    """Rows past 65,536 pools (256-pool groups in the scoring lists) at the
    fewest tokens that reach them: two sequences of 65,537 and 70,000 pools,
    queried at 65,537 pools (a last group of one pool), 65,536 (the last row
    of 64-pool groups), 65,792 (a full last 256-pool group), 70,000 and
    20,000 pools, with tails of 0 to 3 tokens."""
    fv = [1, 3]
    v = [4 * 65537 + 2, 4 * 70000 + 1]
    sl = [a + b for a, b in zip(fv, v)]
    qs = [0, 0, 1, 1, 1]
    qp = [sl[0] - 1, fv[0] + 4 * 65536 + 1, fv[1] + 4 * 65792 - 1, sl[1] - 1, fv[1] + 4 * 20000]
    return _mk("mini_long", seed, production_dims(16), fv, sl, 280004, 70001, qs, qp)


def _with_drafts(wl: Workload, name: str, k: int = 4, note: str = "") -> Workload:
    """The same sequences, each issuing k queries at its last k positions (a
    speculative decode step: the accepted token and k - 1 drafts, scored
    together), queries of one sequence consecutive."""
    qs, qp = [], []
    for b in range(wl.B):
        for i in range(k):
            qs.append(b)
            qp.append(int(wl.seq_len[b]) - k + i)
    return dataclasses.replace(wl, name=name, q_seq=np.asarray(qs, dtype=np.int32),
                               q_pos=np.asarray(qp, dtype=np.int32), note=note)


def mini_mtp(seed: int = 15) -> Workload:
    """mini_decode's sequences with 4 queries each at their last 4 positions."""
    fv = [0, 1, 3, 2]
    v = [4096, 3001, 2050, 517]
    sl = [a + b for a, b in zip(fv, v)]
    base = _mk("mini_mtp", seed, production_dims(16), fv, sl, 4100, 1025, [0], [0])
    return _with_drafts(base, "mini_mtp", 4, "4 queries per sequence (1 + 3 drafts)")


def decode_262k_b8_mtp(seed: int = 2) -> Workload:
    """decode_262k_b8's eight ragged sequences, each issuing 4 queries (the
    accepted token and 3 drafts) at its last 4 positions: 32 queries."""
    return _with_drafts(decode_262k_b8(seed), "decode_262k_b8_mtp", 4, "4 queries per sequence (1 + 3 drafts)")


WORKLOADS = {
    "tiny": tiny, "tiny_seven": tiny_seven, "tiny_padded_six": tiny_padded_six,
    "tiny_batch": tiny_batch,
    "decode_32k": decode_32k, "decode_262k_b8": decode_262k_b8,
    "decode_262k_b8_full": decode_262k_b8_full,
    "prefill_4k_on_131k": prefill_4k_on_131k, "decode_1m_b4": decode_1m_b4,
    "mini_decode": mini_decode, "mini_decode_64": mini_decode_64, "mini_prefill": mini_prefill,
    "mini_heavy": mini_heavy, "mini_mtp": mini_mtp, "decode_262k_b8_mtp": decode_262k_b8_mtp,
    "mini_long": mini_long, "mini_prefill_wide": mini_prefill_wide,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()


# ----------------------------------------------------------------------------
# parallel block generation (large contexts)
# ----------------------------------------------------------------------------

def gen_sequence_blocks(fn, wl: Workload, b: int, x0: int, x1: int, workers: int = 8, step: int = 65536):
    """Yield (x, arrays) chunks of fn(wl, b, x, x+step) over [x0, x1), generated by a thread pool.

    numpy's Philox fills release the GIL, so blocks generate in parallel."""
    import concurrent.futures as cf
    starts = list(range(x0, x1, step))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(fn, wl, b, s, min(s + step, x1)) for s in starts]
        for s, fu in zip(starts, futs):
            yield s, fu.result()


# ----------------------------------------------------------------------------
# synthetic score rows and index lists (inputs for stage-isolated tests)
# ----------------------------------------------------------------------------

def gen_score_rows(seed: int, T: int, stride: int, n_vis: np.ndarray, kind: str = "ties") -> np.ndarray:
    """Float32 score rows [T, stride]; entries past n_vis[t] are -inf.

    kind: "ties" (values on a coarse grid so many scores tie), "normal",
    "equal" (all visible scores equal), "signed_zero" (+0/-0 and small
    negatives)."""
    out = np.full((T, stride), -np.inf, dtype=np.float32)
    for t in range(T):
        g = _rng(seed, "queries", t, 7)
        n = int(n_vis[t])
        if kind == "ties":
            v = np.round(g.standard_normal(n) * 8.0) / 4.0 + 10.0
        elif kind == "normal":
            v = g.standard_normal(n) * 3.0 + 20.0
        elif kind == "equal":
            v = np.full(n, 1.5)
        elif kind == "signed_zero":
            v = np.where(g.random(n) < 0.5, 0.0, -0.0)
            v = np.where(g.random(n) < 0.3, -np.round(g.random(n) * 4) / 4, v)
        else:
            raise ValueError(kind)
        out[t, :n] = v.astype(np.float32)
    return out


def gen_index_lists(seed: int, T: int, width: int, candidates: np.ndarray, valid: np.ndarray,
                    interior_gaps: bool = True) -> np.ndarray:
    """int32 [T, width] lists of distinct rows drawn from `candidates`: valid[t] entries, -1 elsewhere.

    With interior_gaps, the -1 entries are scattered among the valid ones (the
    attention contract skips negative entries wherever they sit)."""
    candidates = np.asarray(candidates, dtype=np.int64)
    out = np.full((T, width), -1, dtype=np.int32)
    for t in range(T):
        g = _rng(seed, "queries", t, 9)
        k = int(valid[t])
        if k == 0:
            continue
        rows = np.sort(g.choice(candidates, size=k, replace=False)).astype(np.int32)
        if interior_gaps and k < width:
            slots = np.sort(g.choice(width, size=k, replace=False))
            out[t, slots] = rows
        else:
            out[t, :k] = rows
    return out


def valid_rows(wl: Workload) -> np.ndarray:
    """Cache rows of every non-padding position of the workload."""
    return np.concatenate([np.arange(int(wl.first_valid[b]), int(wl.seq_len[b])) + int(wl.row_base[b])
                           for b in range(wl.B)]).astype(np.int64)
