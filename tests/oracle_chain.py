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
    def __init__(self, wl: syn.Workload):
        self.wl = wl
        self.d = wl.dims
        self._pools = {}
        self._stored = {}

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
            n_b = int(wl.seq_len[b])
            ks = [int(k) for k in np.unique(pos // blk)]
            with cf.ThreadPoolExecutor(max_workers=8) as ex:
                blocks = ex.map(lambda k: syn.gen_latent(wl, int(b), k * blk, min(n_b, (k + 1) * blk)), ks)
                for k, block in zip(ks, blocks):
                    m = (pos // blk) == k
                    lat[m] = block[pos[m] - k * blk]
            codes, scales = O.quantize_rows(lat)
            out[sel] = O.pack_rows(codes, scales, self.d.row_bytes)
        return out

    def query(self, t: int, stride: int | None = None):
        """Dict with the oracle's scores, pool ids, index list and attention for query t."""
        wl, d = self.wl, self.d
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        n_vis = O.visible_pool_count(qp, f, d.kpool)
        pools = self.pools_stored(b)
        qi = syn.gen_qidx(wl, t, t + 1)[0]
        w = syn.gen_w(wl, t, t + 1)[0]
        scores = O.index_scores(qi, w, pools, n_vis, stride)
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
