"""Decode-step throughput of the DSA path on one MI355X.

One step = the whole path for one batch: store the B new tokens' INT8 rows,
build the pools they complete, score every visible pool, select the top-k,
expand to index lists, and run sparse MLA -- for B = 8 ragged sequences at up
to 262,144 tokens of context, 16 MLA heads.  Inputs are seeded synthetic data
resident in HBM; steps rotate over R replicas of the caches so the working
set exceeds the 256 MB Infinity Cache several times over.

Prints one JSON line (metric, value, ... , roofline, cpu_baseline).
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
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
WORKLOAD = "decode_262k_b8"
_CSRC = os.path.join(ROOT, "sparse_attention_store_amd", "csrc")
SCORES_SRC = [os.path.join(_CSRC, f) for f in ("index_scores.hip", "scores_core.h", "topk_core.h", "new_tokens.h", "dsa_common.h")]
STEP_SRC = [os.path.join(_CSRC, f) for f in ("decode_step.hip", "mla_core.h", "scores_core.h", "topk_core.h",
                                             "dsa_common.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "index_scores_decode_262k_b8_traffic.md")
PMC_SUMMARY_STEP = os.path.join(ROOT, "profiles", "decode_step_decode_262k_b8_traffic.md")
EV_EVERY = 8                    # timed steps between two event-bracketed kernel samples
COPY_BYTES = 256 << 20          # calibration copy: bytes read (and written) per launch


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per decode step (see the design notes)."""
    d = wl.dims
    tot_pools = 0
    tot_rows = 0
    new_pools = 0
    for t in range(wl.T):
        n_vis = wl.n_vis(t)
        b = int(wl.q_seq[t])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        tot_pools += n_vis
        tail = (qp - f + 1) - d.kpool * n_vis if qp >= f else 0
        tot_rows += d.kpool * min(d.select_k, n_vis) + tail
        new_pools += 1 if qp >= f and (qp - f + 1) % d.kpool == 0 else 0
    T = wl.T
    scores = tot_pools * (256 + 4) + T * (d.idx_heads * d.idx_dim * 2 + d.idx_heads * 4)
    step = (tot_pools * 256 + T * (d.idx_heads * d.idx_dim * 2 + d.idx_heads * 4) + tot_rows * d.row_bytes
            + T * 4 * d.mla_heads * d.latent_dim + T * 4 * d.out_width + T * (2 * d.latent_dim + d.row_bytes)
            + new_pools * (2 * d.kpool * d.idx_dim * 2 + d.idx_dim * 2))
    new_tokens = T * (2 * d.latent_dim + d.row_bytes) + new_pools * (2 * d.kpool * d.idx_dim * 2 + d.idx_dim * 2)
    return {"step": step, "scores_kernel": scores + new_tokens, "decode_kernel": step - new_tokens,
            "pools": tot_pools, "rows": tot_rows}


def _source_hash(srcs) -> str:
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(summary: str, srcs):
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3
    counter summary, or None when the summary is absent or was taken on
    different kernel sources."""
    if not os.path.exists(summary):
        return None
    src_hash = _source_hash(srcs)
    vals = {}
    for ln in open(summary):
        if ":" in ln and ln.strip().startswith("- "):
            k, v = ln.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip()
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
    h = _source_hash(STEP_SRC if "decode_step" in kernel else SCORES_SRC)
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


def cpu_baseline(wl, budget_s: float = 12.0) -> dict:
    """The oracle's per-step chain (scores, top-k, expand, attention) for every query of
    the workload, timed on the host cores over whole decode steps.

    Setup (not timed): pools of every sequence (O2, stored bf16) and the INT8 rows
    (O1) of the rows each query's list selects."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import dsa_synth as syn
    import oracle as O

    d = wl.dims
    lw, lb = syn.gen_ln(wl)
    state = []
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        n = int(wl.seq_len[b])
        f = int(wl.first_valid[b])
        qp = int(wl.q_pos[t])
        k = np.empty((n, d.idx_dim), np.float32)
        g = np.empty((n, d.idx_dim), np.float32)
        for x0, (kk, gg) in syn.gen_sequence_blocks(syn.gen_kgate, wl, b, 0, n):
            k[x0:x0 + kk.shape[0]] = kk
            g[x0:x0 + gg.shape[0]] = gg
        pools = O.store_bf16(O.pool_states(k, g, lw, lb, d.ln_eps, f, n, d.kpool))
        del k, g
        qi, w, q = syn.gen_qidx(wl, t, t + 1)[0], syn.gen_w(wl, t, t + 1)[0], syn.gen_q(wl, t, t + 1)[0]
        n_vis = O.visible_pool_count(qp, f, d.kpool)
        idx = O.expand_selection(O.topk_pools(O.index_scores(qi, w, pools, n_vis), n_vis, d.select_k),
                                 f, qp, 0, d.kpool, d.out_width)
        need = idx[idx >= 0]
        rows = np.zeros((n, d.row_bytes), dtype=np.uint8)      # only the listed rows are filled
        blocks = sorted(set(int(x) // 65536 for x in need))
        for blk in blocks:
            lat = syn.gen_latent(wl, b, blk * 65536, min(n, (blk + 1) * 65536))
            sel = need[(need >= blk * 65536) & (need < (blk + 1) * 65536)]
            O.store_int8(lat[sel - blk * 65536], sel, rows)
        state.append((f, qp, n_vis, pools, rows, qi, w, q))
    steps = 0
    t0 = time.perf_counter()
    while True:
        for f, qp, n_vis, pools, rows, qi, w, q in state:
            sc = O.index_scores(qi, w, pools, n_vis)
            ids = O.topk_pools(sc, n_vis, d.select_k)
            idx = O.expand_selection(ids, f, qp, 0, d.kpool, d.out_width)
            O.sparse_mla(q, rows, idx, wl.scale, d.latent_dim)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": steps * wl.T / el, "unit": "tok-steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} whole decode steps ({wl.T} queries each) of {wl.name}: oracle scores, "
                      f"top-k, expansion and attention in float64, {el:.1f} s; pool and INT8-row setup "
                      "not timed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--path", choices=["fused", "separate"], default="separate",
                    help="fused: new tokens, then one dsa_decode_step launch; separate: one call per step")
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
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import dsa_harness
    import dsa_synth as syn

    wl = syn.get(args.workload)
    print(f"[bench] setting up {wl.name}: B={wl.B} T={wl.T} rows={wl.total_rows} "
          f"replicas={args.replicas}", file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    fused = args.path == "fused"
    dw = dsa_harness.DeviceWorkload(wl, replicas=args.replicas, out_dtype=torch.bfloat16,
                                    num_splits=17 if fused else 0)
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    R = args.replicas
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
    # The timed loop launches through prepared calls (validated and converted
    # once per replica): each launch then costs one ctypes call on the host, so
    # the host keeps ahead of the GPU.
    timed_stages = ["append", "decode"] if fused else ["append_scores", "select_attention"]
    for r in range(R):
        for st in timed_stages:
            dw.bound(st, r)
    for i in range(args.warmup):
        for st in timed_stages:
            dw.run(st, i % R)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # The dominant kernel is bracketed by HIP events on every EV_EVERY-th timed
    # step only: an event pair costs several microseconds of stream time, which
    # would otherwise be charged to every step.
    sampled = list(range(0, args.steps, EV_EVERY))
    ev_s = {i: torch.cuda.Event(enable_timing=True) for i in sampled}
    ev_e = {i: torch.cuda.Event(enable_timing=True) for i in sampled}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        r = i % R
        if fused:
            dw.run("append", r)
            if i in ev_s:
                ev_s[i].record(stream)
            dw.run("decode", r)
            if i in ev_e:
                ev_e[i].record(stream)
        else:
            if i in ev_s:
                ev_s[i].record(stream)
            dw.run("append_scores", r)
            if i in ev_e:
                ev_e[i].record(stream)
            dw.run("select_attention", r)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    scores_us = float(np.mean([ev_s[i].elapsed_time(ev_e[i]) for i in sampled])) * 1e3

    # Per-stage breakdown (separate, untimed pass).
    stages = {}
    if fused:
        names = ["append_tokens", "decode_step"]
        fns = [lambda r: dw.run("append", r), lambda r: dw.run("decode", r)]
    else:
        names = ["append_scores_groups", "topk_sparse_mla"]
        fns = [lambda r, st=st: dw.run(st, r) for st in timed_stages]
    n_b = min(args.steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n_b)]
    for i in range(n_b):
        evs[i][0].record(stream)
        for j, fn in enumerate(fns):
            fn(i % R)
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    for j, nm in enumerate(names):
        stages[nm] = round(float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3, 2)

    # The dominant kernel's launch duration.  A burst of back-to-back launches
    # of it alone (cycling the replicas, so its pools come from HBM) between
    # one event pair also counts the gaps between launches (avg_launch_us_burst);
    # the scoring launch can record HIP events around the kernel itself
    # (hipExtLaunchKernel), which give its own duration (avg_launch_us).  An
    # event pair around a single launch inside a step also counts that
    # launch's dispatch latency (avg_launch_us_in_step).
    dom_stage = "decode" if fused else "append_scores"
    dom = lambda r: dw.run(dom_stage, r)
    n_burst = 4 * R
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(n_burst):
        dom(i % R)
    b1.record(stream)
    torch.cuda.synchronize()
    burst_us = b0.elapsed_time(b1) * 1e3 / n_burst
    launch_us = burst_us
    if not fused:
        import sparse_attention_store_amd as dsa
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_burst)]
        for a, b in kev:                        # creates the events
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for i in range(n_burst):
            dsa.time_next_scoring_launch(*kev[i])
            dom(i % R)
        torch.cuda.synchronize()
        launch_us = float(np.mean([a.elapsed_time(b) for a, b in kev])) * 1e3

    ab = algorithmic_bytes(wl)
    kern_bytes = ab["decode_kernel"] if fused else ab["scores_kernel"]
    achieved = kern_bytes / (launch_us * 1e-6) / 1e9
    value = wl.T / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tok-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context_cap": 262144,
                   "valid_tokens": [int(a - b) for a, b in zip(wl.seq_len, wl.first_valid)],
                   "mla_heads": wl.dims.mla_heads, "index_topk": wl.dims.index_topk,
                   "out_width": wl.dims.out_width, "replicas": R},
        "pct_hbm_peak": round(100.0 * ab["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "bytes_per_step": ab["step"],
        "roofline": {"kernel": "decode_step (k_decode_step)" if fused else "append_scores_groups (k_scores_groups)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(PMC_SUMMARY_STEP if fused else PMC_SUMMARY,
                                                     STEP_SRC if fused else SCORES_SRC),
                     "algorithmic_bytes_per_launch": kern_bytes, "avg_launch_us": round(launch_us, 2),
                     "avg_launch_us_burst": round(burst_us, 2),
                     "avg_launch_us_in_step": round(scores_us, 2)},
        "path": args.path,
        "stages_us_median": stages,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
