"""Oracle-side expectations for a whole workload (test infrastructure).

Builds, from the seeded generators only, what the oracle says each step of
the path produces for the queries of a dsa_synth.Workload.  Nothing here reads
a GPU result.
"""
from __future__ import annotations

import concurrent.futures as cf

import numpy as np

import dsa_synth as syn
import oracle as O


class OracleWorkload:
    def __init__(self, wl: syn.Workload, block_cache_bytes: int = 1 << 30):
        self.wl = wl
        self.d = wl.dims
        self._pools = {}
        self._stored = {}
        self._blocks = {}                 # (sequence, block) -> latent rows, bounded by block_cache_bytes
        self._block_cap = max(1, block_cache_bytes // (syn.ROW_BLOCK * self.d.latent_dim * 4))

    def _latent_block(self, b: int, k: int) -> np.ndarray:
        key = (b, k)
        blk = self._blocks.get(key)
        if blk is None:
            n_b = int(self.wl.seq_len[b])
            blk = syn.gen_latent(self.wl, b, k * syn.ROW_BLOCK, min(n_b, (k + 1) * syn.ROW_BLOCK))
            if len(self._blocks) >= self._block_cap:
                self._blocks.pop(next(iter(self._blocks)))
            self._blocks[key] = blk
        return blk

    def pools_stored(self, b: int) -> np.ndarray:
        """Pools of sequence b as stored: O2 in fp64, rounded once to bf16."""
        if b not in self._stored:
            self._stored[b] = O.store_bf16(self.pools(b))
        return self._stored[b]

    def pools(self, b: int) -> np.ndarray:
        """fp64 pools of sequence b (whole sequence), from O2."""
        if b not in self._pools:
            wl = self.wl
            n = int(wl.seq_len[b])
            k = np.empty((n, self.d.idx_dim), np.float32)
            g = np.empty((n, self.d.idx_dim), np.float32)
            for x0, (kk, gg) in syn.gen_sequence_blocks(syn.gen_kgate, wl, b, 0, n):
                k[x0:x0 + kk.shape[0]] = kk
                g[x0:x0 + gg.shape[0]] = gg
            lw, lb = syn.gen_ln(wl)
            self._pools[b] = O.pool_states(k, g, lw, lb, self.d.ln_eps, int(wl.first_valid[b]), n, self.d.kpool)
        return self._pools[b]

    def cache_rows(self, rows: np.ndarray) -> np.ndarray:
        """uint8 [len(rows), row_bytes] INT8 rows (O1) for global cache rows.

        Latent rows are generated block by block (each needed block once)."""
        wl = self.wl
        rows = np.asarray(rows, dtype=np.int64)
        out = np.zeros((rows.size, self.d.row_bytes), dtype=np.uint8)
        if rows.size == 0:
            return out
        seq_of = np.searchsorted(wl.row_base, rows, side="right") - 1
        blk = syn.ROW_BLOCK
        for b in np.unique(seq_of):
            sel = np.nonzero(seq_of == b)[0]
            pos = rows[sel] - int(wl.row_base[b])
            lat = np.empty((sel.size, self.d.latent_dim), dtype=np.float32)
            ks = [int(k) for k in np.unique(pos // blk)]
            with cf.ThreadPoolExecutor(max_workers=8) as ex:
                blocks = ex.map(lambda k: self._latent_block(int(b), k), ks)
                for k, block in zip(ks, blocks):
                    m = (pos // blk) == k
                    lat[m] = block[pos[m] - k * blk]
            codes, scales = O.quantize_rows(lat)
            out[sel] = O.pack_rows(codes, scales, self.d.row_bytes)
        return out

    def query(self, t: int, stride: int | None = None, int8_pools=None):
        """Dict with the oracle's scores, pool ids, index list and attention for query t.

        int8_pools: (codes, scales) of the sequence's pools in the INT8 form;
        the scores are then O3q over them (else O3 over the stored bf16 pools)."""
        wl, d = self.wl, self.d
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        n_vis = O.visible_pool_count(qp, f, d.kpool)
        qi = syn.gen_qidx(wl, t, t + 1)[0]
        w = syn.gen_w(wl, t, t + 1)[0]
        if int8_pools is not None:
            scores = O.index_scores_int8(qi, w, int8_pools[0], int8_pools[1], n_vis, stride)
        else:
            scores = O.index_scores(qi, w, self.pools_stored(b), n_vis, stride)
        ids = O.topk_pools(scores, n_vis, d.select_k)
        idx = O.expand_selection(ids, f, qp, int(wl.row_base[b]), d.kpool, d.out_width)
        valid = idx[idx >= 0]
        rows = self.cache_rows(valid)
        q = syn.gen_q(wl, t, t + 1)[0]
        # Attention over the listed rows: a compact cache holding just those rows.
        local = np.arange(valid.size)
        o, lse = O.sparse_mla(q, rows, local, wl.scale, d.latent_dim) if valid.size else \
            (np.zeros((d.mla_heads, d.latent_dim)), np.full(d.mla_heads, -np.inf))
        return dict(n_vis=n_vis, scores=scores, ids=ids, indices=idx, out=o, lse=lse)


def topk_set_ok(gpu_ids: np.ndarray, oracle_scores: np.ndarray, oracle_ids: np.ndarray, n_vis: int,
                rel: float = 1e-3):
    """End-to-end selection check: sets may differ only among near-ties of the k-th score.

    Returns (ok, n_swapped)."""
    a = set(int(x) for x in gpu_ids if x >= 0)
    bset = set(int(x) for x in oracle_ids if x >= 0)
    if len(a) != len(bset):
        return False, -1
    diff = a ^ bset
    if not diff:
        return True, 0
    k = len(bset)
    s = oracle_scores[:n_vis]
    order = np.lexsort((np.arange(n_vis), -s))
    sk = s[order[k - 1]]
    tol = rel * abs(sk)
    ok = all(p < n_vis and abs(s[p] - sk) <= tol for p in diff)
    return ok, len(diff) // 2


def score_close(gpu: np.ndarray, ref: np.ndarray, n_vis: int, rtol: float = 1e-2, floor: float = 1e-2):
    """Elementwise rtol with an absolute floor of floor * RMS of the reference row."""
    g, r = gpu[:n_vis].astype(np.float64), ref[:n_vis]
    if n_vis == 0:
        return True, 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    bound = rtol * np.abs(r) + floor * rms
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)))


# A GPU pool's fp32 state differs from the oracle's fp64 state rounded to fp32
# by a few fp32 rounding steps (LayerNorm, softmax, sums): well under 2^-18 of
# the row's amax, i.e. under 127 * 2^-18 < 5e-4 of one code step.  A code may
# therefore differ from the oracle's by one only where the oracle's x / s lies
# within that distance of a rounding boundary (k + 1/2).
INT8_BOUNDARY = 5e-4


def check_int8_pools(codes: np.ndarray, scales: np.ndarray, opools: np.ndarray, where) -> None:
    """GPU INT8 pools against the oracle's quantiser (O2q) of its fp64 pools."""
    oc, osc = O.quantize_pools(opools)
    assert np.allclose(scales.astype(np.float64), osc.astype(np.float64), rtol=2e-6, atol=0), ("pool scales", where)
    diff = codes.astype(np.int64) - oc.astype(np.int64)
    assert np.all(np.abs(diff) <= 1), ("pool codes", where)
    if np.any(diff):
        ratio = np.asarray(opools, np.float64).astype(np.float32).astype(np.float64) / osc.astype(np.float64)[:, None]
        near = np.abs(np.abs(ratio - np.floor(ratio)) - 0.5) <= INT8_BOUNDARY
        assert np.all(near[diff != 0]), ("pool code off a rounding boundary", where)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (the rounding of a bf16 output)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 8)


def check_chain(dw, queries, pool_sample: int = 64, say=print) -> dict:
    """Every stage of the step dw ran, for each query in `queries`:

    * pools (a sample per sequence) and scores against the oracle's (O2, O3):
      rtol 1e-2 with a floor of 1e-2 x RMS of the oracle row; score tails -inf.
      INT8 pools (dw.int8): codes and scales against the oracle's quantiser
      (check_int8_pools), and the scores against O3q on the GPU's own codes;
    * stage-isolated selection: the oracle's top-k (O4) and expansion (O5) run
      on the GPU's own fp32 score row must reproduce pool_ids and the index
      list bit for bit;
    * end-to-end selection: the GPU's set may differ from the oracle's fp64
      chain only among pools within 1e-3 (relative) of the k-th oracle score;
    * cache rows of the GPU's list: bit-exact against O1;
    * attention: O6 on the GPU's list and cache bytes, max-abs 2e-2 (plus half a
      bf16 ulp of the reference for a bf16 output) and rel-L2 1e-2 over all the
      checked queries; an empty list gives exactly 0 and lse -inf.
    No query is skipped.  Returns counts for the report."""
    import torch
    queries = [int(t) for t in queries]
    wl = dw.wl
    d = wl.dims
    ow = OracleWorkload(wl)
    scores = dw.scores.cpu().numpy()
    ids = dw.pool_ids.cpu().numpy()
    idx = dw.indices.cpu().numpy()
    out_bf16 = dw.out.dtype == torch.bfloat16
    out = dw.out.float().cpu().numpy()
    lse = dw.lse.cpu().numpy()
    int8 = getattr(dw, "int8", False)
    if int8:
        codes = dw.pool_codes[0].cpu().numpy()
        pscales = dw.pool_scales[0].cpu().numpy()
    else:
        pools = dw.pools[0].float().cpu().numpy()
    errs, refs, allow = [], [], []
    near_ties = 0
    g = np.random.default_rng(17)
    checked_pools = set()
    for t in queries:
        t = int(t)
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        say(f"  oracle query {t} (sequence {b}, position {qp})")
        pb = int(wl.pool_base[b])
        if int8:
            # the oracle's scores on the GPU's own INT8 pools (O3q); the codes
            # themselves are checked against the oracle's quantiser below
            n_p = wl.n_pools(b)
            r = ow.query(t, dw.stride, int8_pools=(codes[pb:pb + n_p], pscales[pb:pb + n_p]))
        else:
            r = ow.query(t, dw.stride)
        n_vis = r["n_vis"]
        if b not in checked_pools:
            checked_pools.add(b)
            opools = ow.pools(b)
            sel = np.arange(opools.shape[0]) if opools.shape[0] <= pool_sample else \
                g.choice(opools.shape[0], size=pool_sample, replace=False)
            if int8:
                check_int8_pools(codes[pb + sel], pscales[pb + sel], opools[sel], (t, b))
            else:
                for p in sel:
                    ok, worst = score_close(pools[pb + p], opools[p], d.idx_dim)
                    assert ok, ("pool", t, int(p), worst)
        ok, worst = score_close(scores[t], r["scores"], n_vis)
        assert ok, ("scores", t, worst)
        assert np.all(np.isneginf(scores[t, n_vis:])), ("scores tail", t)
        # stage-isolated: O4 + O5 on the GPU's own scores
        iso_ids = O.topk_pools(scores[t].astype(np.float64), n_vis, d.select_k)
        assert np.array_equal(ids[t], iso_ids), ("pool_ids vs O4 on the GPU scores", t)
        iso_idx = O.expand_selection(iso_ids, f, qp, int(wl.row_base[b]), d.kpool, d.out_width)
        assert np.array_equal(idx[t], iso_idx), ("indices vs O5", t)
        # end-to-end: near-ties only
        ok, nsw = topk_set_ok(ids[t], r["scores"], r["ids"], n_vis)
        assert ok, ("top-k set beyond near-ties", t)
        near_ties += nsw > 0
        # rows of the GPU's own list, then O6 on them
        valid = idx[t][idx[t] >= 0]
        got_rows = dw.caches[0][torch.from_numpy(valid.astype(np.int64)).to(dw.device)].cpu().numpy().view(np.uint8)
        assert np.array_equal(got_rows, ow.cache_rows(valid)), ("rows", t)
        q = syn.gen_q(wl, t, t + 1)[0]
        if valid.size == 0:
            assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t])), ("empty list", t)
            continue
        o_ref, lse_ref = O.sparse_mla(q, got_rows, np.arange(valid.size), wl.scale, d.latent_dim)
        errs.append(out[t] - o_ref)
        refs.append(o_ref)
        allow.append(2e-2 + (bf16_half_ulp(o_ref) if out_bf16 else np.zeros_like(o_ref)))
        assert np.allclose(lse[t], lse_ref, atol=2e-3, rtol=1e-4), ("lse", t)
    if errs:
        e, rf, al = np.stack(errs), np.stack(refs), np.stack(allow)
        assert np.all(np.abs(e) <= al), float(np.max(np.abs(e) - al))
        if np.linalg.norm(rf) > 0:
            assert np.linalg.norm(e) / np.linalg.norm(rf) <= 1e-2
    return {"queries": len(queries), "near_tie_queries": int(near_ties)}
