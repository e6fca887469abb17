"""Throughput of the DSA path on one MI355X.

One step = the whole path for one batch: store the new tokens' INT8 rows,
build the pools they complete, score every visible pool, select the top-k,
expand to index lists, and run sparse MLA.  The default workload is the
decode batch the metric is quoted on: B = 8 ragged sequences at up to
262,144 tokens of context, 16 MLA heads.  --workload picks another
configuration: decode_32k (B = 1), decode_1m_b4 (B = 4 at 1,048,576
positions, 64 heads) or prefill_4k_on_131k (4,096 causal queries on a
131,072-token context, 64 heads, scored 512 queries at a time).  Inputs are
seeded synthetic data resident in HBM; decode steps rotate over R replicas of
the caches so the working set exceeds the 256 MB Infinity Cache several
times over.

Prints one JSON line (metric, value, ..., roofline, cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tok-steps/s (indexer+topk+sparse MLA) @262k ctx B=8; % HBM peak"
METRICS = {
    "decode_262k_b8": METRIC,
    "decode_262k_b8_full": "decode tok-steps/s (indexer+topk+sparse MLA) @262k ctx B=8, all sequences full; % HBM peak",
    "decode_32k": "decode tok-steps/s (indexer+topk+sparse MLA) @32k ctx B=1; % HBM peak",
    "decode_1m_b4": "decode tok-steps/s (indexer+topk+sparse MLA) @1M ctx B=4, 64 heads; % HBM peak",
    "prefill_4k_on_131k": "prefill tokens/s (indexer+topk+sparse MLA), 4096 queries on 131k ctx, 64 heads; % MFMA peak",
    "decode_262k_b8_mtp": "decode tok-steps/s (indexer+topk+sparse MLA) @262k ctx B=8, 4 queries per sequence "
                          "(1 + 3 drafts); % HBM peak",
}
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
WORKLOAD = "decode_262k_b8"
_CSRC = os.path.join(ROOT, "sparse_attention_store_amd", "csrc")
_SCORES_HDR = ("scores_core.h", "scores_decode.h", "topk_core.h", "new_tokens.h", "dsa_common.h")
SCORES_SRC = [os.path.join(_CSRC, f) for f in ("index_scores.hip",) + _SCORES_HDR]
# the sources each profiled kernel is built from (a counter summary names their hash)
KERNEL_SRC = {
    "k_scores_groups": SCORES_SRC,
    "k_scores_runs": [os.path.join(_CSRC, f) for f in ("index_scores_runs.hip",) + _SCORES_HDR],
    "k_scores_mfma": SCORES_SRC,
    "k_select_mla": [os.path.join(_CSRC, f) for f in ("select_mla.hip", "group_select.h", "mla_core.h",
                                                      "topk_core.h", "dsa_common.h")],
    "k_mla_mfma": [os.path.join(_CSRC, f) for f in ("sparse_mla.hip", "mla_core.h", "dsa_common.h")],
    "k_mla_combine": [os.path.join(_CSRC, f) for f in ("sparse_mla.hip", "mla_core.h", "dsa_common.h")],
    "k_decode_step": [os.path.join(_CSRC, f) for f in ("decode_step.hip", "mla_core.h", "scores_core.h",
                                                       "topk_core.h", "dsa_common.h")],
}
# committed counter summaries of the timed scoring launch: (workload, INT8 pools, share) -> (file, block)
TRAFFIC_PROFILES = {
    ("decode_262k_b8", False, 1): ("index_scores_decode_262k_b8_traffic.md", 0),
    ("decode_262k_b8", True, 1): ("index_scores_int8_decode_262k_b8_traffic.md", 0),
    ("decode_1m_b4", False, 1): ("index_scores_decode_1m_b4_traffic.md", 0),
    ("decode_262k_b8_mtp", False, 4): ("index_scores_shared_decode_262k_b8_mtp_traffic.md", 0),
    ("decode_262k_b8_mtp", False, 1): ("index_scores_shared_decode_262k_b8_mtp_traffic.md", 1),
}
COPY_BYTES = 256 << 20          # calibration copy: bytes read (and written) per launch


def algorithmic_bytes(wl, pool_bytes: int = 256, share: int = 1) -> dict:
    """Bytes the method must move per decode step (see the design notes).
    pool_bytes: a stored pool (256 in bf16; 132 as INT8 codes plus an fp32 scale).
    share > 1: runs of up to `share` consecutive queries of one sequence read
    its pools once (the largest visible count of the run)."""
    d = wl.dims
    tot_pools = 0
    tot_rows = 0
    new_pools = 0
    run_len, run_max = 0, 0
    for t in range(wl.T):
        n_vis = wl.n_vis(t)
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        if run_len and b == int(wl.q_seq[t - 1]) and run_len < share:
            run_len += 1
            tot_pools += max(0, n_vis - run_max)
            run_max = max(run_max, n_vis)
        else:
            run_len, run_max = 1, n_vis
            tot_pools += n_vis
        tail = (qp - f + 1) - d.kpool * n_vis if qp >= f else 0
        tot_rows += d.kpool * min(d.select_k, n_vis) + tail
        new_pools += 1 if qp >= f and (qp - f + 1) % d.kpool == 0 else 0
    # the score rows and q_idx are per query, the pools per run
    score_writes = sum(wl.n_vis(t) for t in range(wl.T))
    T = wl.T
    scores = tot_pools * pool_bytes + score_writes * 4 + T * (d.idx_heads * d.idx_dim * 2 + d.idx_heads * 4)
    new_pool_out = d.idx_dim * 2 if pool_bytes == 256 else pool_bytes
    step = (tot_pools * pool_bytes + T * (d.idx_heads * d.idx_dim * 2 + d.idx_heads * 4) + tot_rows * d.row_bytes
            + T * 4 * d.mla_heads * d.latent_dim + T * 4 * d.out_width + T * (2 * d.latent_dim + d.row_bytes)
            + new_pools * (2 * d.kpool * d.idx_dim * 2 + new_pool_out))
    new_tokens = T * (2 * d.latent_dim + d.row_bytes) + new_pools * (2 * d.kpool * d.idx_dim * 2 + new_pool_out)
    return {"step": step, "scores_kernel": scores + new_tokens, "decode_kernel": step - new_tokens,
            "pools": tot_pools, "rows": tot_rows}


def _source_hash(srcs) -> str:
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def device_info() -> dict:
    """What the runtime reports of the GPU the line was measured on (the peaks
    above are the spec sheet's; this confirms the part and its unit counts)."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "l2_bytes": getattr(p, "L2_cache_size", None)}


def traffic_from_profile(summary: str, srcs, block: int = 0):
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3
    counter summary (its block-th kernel summary), or None when the summary is
    absent or was taken on different kernel sources."""
    if not os.path.exists(summary):
        return None
    src_hash = _source_hash(srcs)
    blocks = []
    for ln in open(summary):
        if ":" in ln and ln.strip().startswith("- "):
            k, v = ln.strip()[2:].split(":", 1)
            if k.strip() == "kernel":
                blocks.append({})
            if blocks:
                blocks[-1][k.strip()] = v.strip()
    if block >= len(blocks):
        return None
    vals = blocks[block]
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(files[0])))


def summarize_trace(d: str) -> str:
    """Per-kernel durations of the library's kernels from a rocprofv3 kernel trace."""
    import collections
    import statistics
    by = collections.defaultdict(list)
    for r in _csv_rows(d, "kernel_trace.csv"):
        if "dsa::" in r["Kernel_Name"]:
            by[r["Kernel_Name"].split("(")[0]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | dispatches | mean us | median us | min us |", "|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -statistics.mean(kv[1])):
        out.append(f"| `{k}` | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} |")
    return "\n".join(out)


def summarize_pmc(fetch_dir: str, write_dir: str, kernel: str) -> str:
    """HBM bytes per dispatch of `kernel` from FETCH_SIZE and WRITE_SIZE runs, each scaled by
    what the same counter reads for the calibration copy (COPY_BYTES read and written)."""
    import statistics
    vals = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == name]
        cal = [float(r["Counter_Value"]) * 1024 for r in rows if "neg_kernel" in r["Kernel_Name"]]
        ker = [float(r["Counter_Value"]) * 1024 for r in rows if kernel in r["Kernel_Name"]]
        if not cal or not ker:
            raise SystemExit(f"{name}: calibration copy or kernel {kernel!r} not found")
        factor = COPY_BYTES / statistics.median(cal)
        vals[name] = (statistics.median(ker), factor, len(ker))
    f_raw, f_fac, n_f = vals["FETCH_SIZE"]
    w_raw, w_fac, n_w = vals["WRITE_SIZE"]
    total = f_raw * f_fac + w_raw * w_fac
    h = _source_hash(next((v for k, v in KERNEL_SRC.items() if k in kernel), SCORES_SRC))
    return "\n".join([
        f"- kernel: {kernel}",
        f"- dispatches: {n_f} (FETCH_SIZE run), {n_w} (WRITE_SIZE run)",
        f"- fetch_bytes_raw_median: {f_raw:.0f}",
        f"- fetch_scale_from_copy: {f_fac:.4f}",
        f"- write_bytes_raw_median: {w_raw:.0f}",
        f"- write_scale_from_copy: {w_fac:.4f}",
        f"- hbm_bytes_per_launch: {total:.0f}",
        f"- kernel_source_sha256_16: {h}",
    ])


def prefill_work(wl) -> dict:
    """Algorithmic flops and bytes of one prefill step (all queries)."""
    d = wl.dims
    nvis = 0
    rows = 0
    for t in range(wl.T):
        n_vis = wl.n_vis(t)
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        nvis += n_vis
        tail = (qp - f + 1) - d.kpool * n_vis if qp >= f else 0
        rows += d.kpool * min(d.select_k, n_vis) + tail
    score_flops = 2 * d.idx_heads * d.idx_dim * nvis
    attn_flops = 4 * d.mla_heads * d.latent_dim * rows
    uniq_rows = int(sum(int(wl.seq_len[b]) - int(wl.first_valid[b]) for b in range(wl.B)))
    bytes_ = (wl.T * (d.idx_heads * d.idx_dim * 2 + d.idx_heads * 4) + wl.total_pools * 256
              + wl.T * 4 * d.mla_heads * d.latent_dim + wl.T * 4 * d.out_width + uniq_rows * d.row_bytes)
    return {"score_flops": score_flops, "attn_flops": attn_flops, "sum_n_vis": nvis, "rows": rows, "bytes": bytes_}


def _oracle_state(wl, t, O, syn, d, lw, lb, pools_cache, rows_cache, int8=False):
    """Per-query oracle inputs (not timed): the sequence's pools (O2, stored bf16,
    or with int8 as codes and scales, O2q) and the INT8 rows (O1) of the
    positions the query's list selects."""
    import numpy as np
    b = int(wl.q_seq[t])
    n = int(wl.seq_len[b])
    f = int(wl.first_valid[b])
    qp = int(wl.q_pos[t])
    if b not in pools_cache:
        k = np.empty((n, d.idx_dim), np.float32)
        g = np.empty((n, d.idx_dim), np.float32)
        for x0, (kk, gg) in syn.gen_sequence_blocks(syn.gen_kgate, wl, b, 0, n):
            k[x0:x0 + kk.shape[0]] = kk
            g[x0:x0 + gg.shape[0]] = gg
        ps = O.pool_states(k, g, lw, lb, d.ln_eps, f, n, d.kpool)
        pools_cache[b] = O.quantize_pools(ps) if int8 else O.store_bf16(ps)
        del k, g
    pools = pools_cache[b]
    qi, w, q = syn.gen_qidx(wl, t, t + 1)[0], syn.gen_w(wl, t, t + 1)[0], syn.gen_q(wl, t, t + 1)[0]
    n_vis = O.visible_pool_count(qp, f, d.kpool)
    sc = O.index_scores_int8(qi, w, pools[0], pools[1], n_vis) if int8 else O.index_scores(qi, w, pools, n_vis)
    idx = O.expand_selection(O.topk_pools(sc, n_vis, d.select_k), f, qp, 0, d.kpool, d.out_width)
    need = idx[idx >= 0]
    if b not in rows_cache:
        rows_cache[b] = (np.zeros((n, d.row_bytes), dtype=np.uint8), set())
    rows, done = rows_cache[b]
    blk = 65536
    for k0 in sorted(set(int(x) // blk for x in need) - done):
        lat = syn.gen_latent(wl, b, k0 * blk, min(n, (k0 + 1) * blk))
        O.store_int8(lat, np.arange(k0 * blk, k0 * blk + lat.shape[0]), rows)
        done.add(k0)
    return (f, qp, n_vis, pools, rows, qi, w, q)


def cpu_baseline(wl, budget_s: float = 12.0, max_queries: int | None = None, int8: bool = False) -> dict:
    """The oracle's per-query chain (scores, top-k, expansion, attention), timed
    on the host cores: whole decode steps (every query of the batch) for decode
    workloads, a seeded sample of queries for prefill.  Setup (pools of every
    sequence, O2; INT8 rows, O1) is not timed.  Timed twice: with the BLAS
    threads set to the cores this process may run on, then with one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import dsa_synth as syn
    import oracle as O

    d = wl.dims
    lw, lb = syn.gen_ln(wl)
    if max_queries is not None and wl.T > max_queries:
        g = np.random.default_rng(7)
        queries = sorted(int(x) for x in g.choice(wl.T, size=max_queries, replace=False))
    else:
        queries = list(range(wl.T))
    pools_cache, rows_cache = {}, {}
    state = [_oracle_state(wl, t, O, syn, d, lw, lb, pools_cache, rows_cache, int8) for t in queries]

    def run(limit_s):
        passes = 0
        t0 = time.perf_counter()
        while True:
            for f, qp, n_vis, pools, rows, qi, w, q in state:
                sc = O.index_scores_int8(qi, w, pools[0], pools[1], n_vis) if int8 else \
                    O.index_scores(qi, w, pools, n_vis)
                ids = O.topk_pools(sc, n_vis, d.select_k)
                idx = O.expand_selection(ids, f, qp, 0, d.kpool, d.out_width)
                O.sparse_mla(q, rows, idx, wl.scale, d.latent_dim)
            passes += 1
            el = time.perf_counter() - t0
            if el >= limit_s:
                return passes * len(state) / el, passes, el

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        v, passes, el = run(budget_s)
    with threadpool_limits(limits=1):
        v1, passes1, el1 = run(budget_s / 2)
    prefill = wl.T > 64
    unit = "tok/s" if prefill else "tok-steps/s"
    what = (f"{passes} passes over a seeded sample of {len(state)} of the {wl.T} prefill queries"
            if len(state) < wl.T else f"{passes} whole decode steps ({wl.T} queries each)")
    return {"value": v, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{what} of {wl.name}: oracle scores{' over INT8 pools' if int8 else ''}, top-k, expansion "
                      f"and attention in float64, "
                      f"{el:.1f} s with {cores} BLAS threads; pool and INT8-row setup not timed",
            "value_1thread": v1, "sample_1thread": f"{passes1} passes, {el1:.1f} s, 1 thread"}


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def copy_rate_gbs(reps: int = 10) -> float:
    """A plain device copy of COPY_BYTES (read + write), the practical HBM ceiling."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = _ev(), _ev()
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * COPY_BYTES * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def _pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def time_steps(dw, steps: int, warmup: int, R: int, group: int):
    """Warm up, then time `steps` steps (stages dw.timed_stages(), replica i % R)
    bracketed by one event pair; an event between every `group` steps gives the
    per-step spread (median, p10, p90 of the group means)."""
    import torch
    stages = dw.timed_stages()
    for r in range(R):
        for st in stages:
            dw.bound(st, r)
    for i in range(warmup):
        dw.step_timed(i % R)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    marks = [_ev() for _ in range(steps // group + 2)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    k = 1
    for i in range(steps):
        dw.step_timed(i % R)
        if (i + 1) % group == 0 or i + 1 == steps:
            marks[k].record(stream)
            k += 1
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[k - 1])
    per = []
    done = 0
    for j in range(1, k):
        n = min(group, steps - done)
        per.append(marks[j - 1].elapsed_time(marks[j]) * 1e3 / n)
        done += n
    return total_ms / steps, per


def stage_breakdown(dw, R: int, n: int):
    """Median time of each stage inside a step (events between the stages, an
    untimed pass)."""
    import numpy as np
    import torch
    stages = dw.timed_stages()
    stream = torch.cuda.current_stream()
    evs = [[_ev() for _ in range(len(stages) + 1)] for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        for j, st in enumerate(stages):
            dw.run(st, i % R)
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return {st: round(float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3, 2)
            for j, st in enumerate(stages)}


def scoring_launch_us(dw, R: int, n: int):
    """The decode scoring kernel's own duration: HIP events recorded around the
    kernel itself (dsa_time_next_scoring_launch), over n launches of its stage
    alone cycling the replicas (mean); plus the same n launches back to back
    between one event pair (burst, which also counts the gaps)."""
    import numpy as np
    import torch
    import sparse_attention_store_amd as dsa
    stage = dw.timed_stages()[0] if dw.fast_supported() else "scores_select"
    stream = torch.cuda.current_stream()
    b0, b1 = _ev(), _ev()
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(n):
        dw.run(stage, i % R)
    b1.record(stream)
    torch.cuda.synchronize()
    burst = b0.elapsed_time(b1) * 1e3 / n
    kev = [(_ev(), _ev()) for _ in range(n)]
    for a, b in kev:                        # creates the events
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(n):
        dsa.time_next_scoring_launch(*kev[i])
        dw.run(stage, i % R)
    torch.cuda.synchronize()
    own = [a.elapsed_time(b) * 1e3 for a, b in kev]
    return float(np.mean(own)), float(np.median(own)), burst


def prefill_kernel_us(dw, reps: int = 3):
    """Durations of the prefill's two MFMA kernels: the scoring kernel on one
    chunk of dw.prefill_chunk queries (events recorded around the kernel itself),
    and the attention launch over all queries (an event pair around the call;
    at milliseconds per launch the pair's own cost is negligible)."""
    import numpy as np
    import torch
    import sparse_attention_store_amd as dsa
    c = dw.prefill_chunk
    sc = torch.empty((c, dw.stride), dtype=torch.float32, device=dw.device)
    stream = torch.cuda.current_stream()
    kev = [(_ev(), _ev()) for _ in range(reps)]
    for a, b in kev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    # the chunk in the middle of the prefill (its average visible pool count)
    t0 = (dw.wl.T // c // 2) * c
    args = (dw.dims, dw.q_idx[t0:t0 + c], dw.w[t0:t0 + c], dw.pools[0], dw.seqs, dw.q_seq[t0:t0 + c],
            dw.q_pos[t0:t0 + c], sc)
    for a, b in kev:
        dsa.time_next_scoring_launch(a, b)
        dsa.index_scores(*args)
    torch.cuda.synchronize()
    score_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in kev]))
    chunk_nvis = sum(dw.wl.n_vis(t) for t in range(t0, t0 + c))
    a, b = _ev(), _ev()
    dw.run("attention", 0)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        dw.run("attention", 0)
    b.record(stream)
    torch.cuda.synchronize()
    attn_us = a.elapsed_time(b) * 1e3 / reps
    del sc
    return score_us, chunk_nvis, attn_us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 200 decode, 10 prefill)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 20 decode, 2 prefill)")
    ap.add_argument("--replicas", type=int, default=None, help="cache replicas cycled by the steps (default 8 decode, "
                                                               "1 prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(METRICS))
    ap.add_argument("--share", type=int, default=None,
                    help="queries per run sharing one pass over a sequence's pools (1-4; default 4 for the "
                         "4-queries-per-sequence workload, else 1)")
    ap.add_argument("--pools", default="bf16", choices=["bf16", "int8"],
                    help="pool cache format: bf16 rows (the metric's configuration) or INT8 codes with an fp32 "
                         "scale per pool (decode workloads of at most 65,536 pools per sequence)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB elementwise copy (torch.neg) three times: a "
                         "known-size kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of DIR/*kernel_trace.csv (rocprofv3 --kernel-trace) and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print a markdown traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--kernel", default="k_scores_groups", help="kernel name substring for --summarize-pmc")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.kernel))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (no multi-GPU path exists)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import dsa_harness
    import dsa_synth as syn

    wl = syn.get(args.workload)
    prefill = wl.T > 64
    steps = args.steps if args.steps is not None else (10 if prefill else 200)
    warmup = args.warmup if args.warmup is not None else (2 if prefill else 20)
    R = args.replicas if args.replicas is not None else (1 if prefill else 8)
    print(f"[bench] setting up {wl.name}: B={wl.B} T={wl.T} rows={wl.total_rows} replicas={R}",
          file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    int8 = args.pools == "int8"
    share = args.share if args.share is not None else (4 if wl.name.endswith("_mtp") else 1)
    dw = dsa_harness.DeviceWorkload(wl, replicas=R, out_dtype=torch.bfloat16, pool_format=args.pools, share=share)
    if int8 and not dw.fast_supported():
        raise SystemExit("--pools int8 covers decode workloads of at most 64 queries and 65,536 pools per sequence")
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; stages {dw.timed_stages()}",
          file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
    copy_gbs = copy_rate_gbs()
    ms_step, per_step_us = time_steps(dw, steps, warmup, R, group=R if not prefill else 1)
    stages = stage_breakdown(dw, R, min(steps, 50 if not prefill else 5))
    value = wl.T / (ms_step * 1e-3)
    line = {
        "metric": METRICS[wl.name] + ("; INT8 pool cache" if int8 else ""),
        "value": round(value, 1),
        "unit": "tok/s" if prefill else "tok-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "queries": wl.T,
                   "context_cap": int(wl.row_base[1] - wl.row_base[0]) if wl.B > 1 else int(wl.seq_len[0]),
                   "valid_tokens": [int(a - b) for a, b in zip(wl.seq_len, wl.first_valid)][:16],
                   "mla_heads": wl.dims.mla_heads, "index_topk": wl.dims.index_topk,
                   "out_width": wl.dims.out_width, "replicas": R, "pool_cache": args.pools, "share": share},
        "step_us": {"mean": round(ms_step * 1e3, 2), "median": round(_pct(per_step_us, 50), 2),
                    "p10": round(_pct(per_step_us, 10), 2), "p90": round(_pct(per_step_us, 90), 2),
                    "samples": len(per_step_us), "steps_per_sample": R if not prefill else 1},
        "copy_gbs": round(copy_gbs, 1),
        "stages_us_median": stages,
        "device": device_info(),
    }
    if prefill:
        pw = prefill_work(wl)
        score_us, chunk_nvis, attn_us = prefill_kernel_us(dw)
        chunk_flops = 2 * wl.dims.idx_heads * wl.dims.idx_dim * chunk_nvis
        n_chunks = -(-wl.T // dw.prefill_chunk)
        s_tf = chunk_flops / (score_us * 1e-6) / 1e12
        a_tf = pw["attn_flops"] / (attn_us * 1e-6) / 1e12
        kernels = {
            "index_scores (k_scores_mfma<4,2>), one 512-query chunk": {
                "avg_launch_us": round(score_us, 1), "flops_per_launch": chunk_flops,
                "achieved_tflops": round(s_tf, 1), "frac": round(s_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "launches_per_step": n_chunks},
            "sparse_mla (k_mla_mfma<4, 8>)": {
                "avg_launch_us": round(attn_us, 1), "flops_per_launch": pw["attn_flops"],
                "achieved_tflops": round(a_tf, 1), "frac": round(a_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "launches_per_step": 1},
        }
        dom_attn = attn_us >= score_us * n_chunks
        line["pct_mfma_peak"] = round(100.0 * (pw["score_flops"] + pw["attn_flops"]) / (ms_step * 1e-3) / 1e12
                                      / MFMA_BF16_PEAK_TFLOPS, 2)
        line["flops_per_step"] = pw["score_flops"] + pw["attn_flops"]
        line["roofline"] = {
            "kernel": "sparse_mla (k_mla_mfma<4, 8>)" if dom_attn else "index_scores (k_scores_mfma<4,2>)",
            "bound": "mfma", "achieved": round(a_tf if dom_attn else s_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round((a_tf if dom_attn else s_tf) / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "flops_per_launch": pw["attn_flops"] if dom_attn else chunk_flops,
            "avg_launch_us": round(attn_us if dom_attn else score_us, 1)}
        line["kernels"] = kernels
    else:
        ab = algorithmic_bytes(wl, 132 if int8 else 256, share)
        fast = dw.fast_supported()
        kern_bytes = ab["scores_kernel"] if fast else ab["scores_kernel"] - (ab["step"] - ab["decode_kernel"])
        prof = TRAFFIC_PROFILES.get((wl.name, bool(int8), share))
        own_mean, own_median, burst = scoring_launch_us(dw, R, 4 * R)
        achieved = kern_bytes / (own_mean * 1e-6) / 1e9
        line["pct_hbm_peak"] = round(100.0 * ab["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
        line["bytes_per_step"] = ab["step"]
        line["roofline"] = {
            "kernel": ("append_scores_groups_shared (k_scores_runs<true, 512, %s>)" % ("true" if int8 else "false")
                       if share > 1 else
                       "append_scores_groups_int8 (k_scores_groups<true, 512, true>)" if int8 else
                       "append_scores_groups (k_scores_groups<true, 512, false, false, %s>)"
                       % ("true" if dw.stride > 65536 else "false") if fast else
                       "index_scores_select (k_scores_groups<false, 0, false>)"),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (traffic_from_profile(os.path.join(ROOT, "profiles", prof[0]),
                                             KERNEL_SRC["k_scores_runs" if share > 1 else "k_scores_groups"], prof[1])
                        if fast and prof else None),
            "algorithmic_bytes_per_launch": kern_bytes, "avg_launch_us": round(own_mean, 2),
            "median_launch_us": round(own_median, 2), "avg_launch_us_burst": round(burst, 2),
            "frac_of_copy": round(achieved / copy_gbs, 4)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, max_queries=32 if prefill else None, int8=int8)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
