"""End-to-end parity of the whole path (GPU) against the oracle chain.

The GPU runs the step exactly as the bench does (dsa_harness.DeviceWorkload);
the oracle recomputes everything from the seeded generators.  Checks:
  * INT8 rows of every listed cache row: bit-exact;
  * pools and scores: rtol 1e-2 with an absolute floor of 1e-2 x row RMS;
  * selected pool sets: equal, or differing only among pools whose oracle
    score lies within 1e-3 (relative) of the k-th oracle score;
  * index lists: bit-exact whenever the selected sets agree;
  * attention (fp32 out): max-abs 2e-2 and rel-L2 1e-2 over the workload,
    on every query whose list agrees with the oracle's.
Reduced-size workloads are checked on every output; the full-size workloads
(the pages' shapes) on every decode query and a seeded sample of prefill
queries.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import dsa_synth as syn
from oracle_chain import OracleWorkload, score_close, topk_set_ok

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_harness
    return dsa_harness


def _check_chain(dw, queries, pool_sample=64, allow_swaps_frac=0.05):
    wl = dw.wl
    d = wl.dims
    ow = OracleWorkload(wl)
    scores = dw.scores.cpu().numpy()
    ids = dw.pool_ids.cpu().numpy()
    idx = dw.indices.cpu().numpy()
    out = dw.out.float().cpu().numpy()
    lse = dw.lse.cpu().numpy()
    pools = dw.pools[0].float().cpu().numpy()
    errs, refs = [], []
    swapped = 0
    g = np.random.default_rng(17)
    for t in queries:
        b = int(wl.q_seq[t])
        say(f"  oracle query {int(t)} (sequence {b}, position {int(wl.q_pos[t])})")
        r = ow.query(int(t), dw.stride)
        n_vis = r["n_vis"]
        # pools of this sequence (a sample at full size)
        pb = int(wl.pool_base[b])
        opools = ow.pools(b)
        sel = np.arange(opools.shape[0]) if opools.shape[0] <= pool_sample else \
            g.choice(opools.shape[0], size=pool_sample, replace=False)
        for p in sel:
            ok, worst = score_close(pools[pb + p], opools[p], d.idx_dim)
            assert ok, ("pool", t, int(p), worst)
        ok, worst = score_close(scores[t], r["scores"], n_vis)
        assert ok, ("scores", t, worst)
        assert np.all(np.isneginf(scores[t, n_vis:])), ("scores tail", t)
        ok, nsw = topk_set_ok(ids[t], r["scores"], r["ids"], n_vis)
        assert ok, ("topk", t)
        assert np.all(ids[t][min(d.select_k, n_vis):] == -1)
        assert np.all(np.diff(ids[t][:min(d.select_k, n_vis)]) > 0)
        if nsw:
            swapped += 1
            continue
        assert np.array_equal(ids[t], r["ids"]), ("ids", t)
        assert np.array_equal(idx[t], r["indices"]), ("indices", t)
        valid = idx[t][idx[t] >= 0]
        got_rows = dw.caches[0][torch.from_numpy(valid.astype(np.int64)).cuda()].cpu().numpy().view(np.uint8)
        assert np.array_equal(got_rows, ow.cache_rows(valid)), ("rows", t)
        errs.append(out[t] - r["out"])
        refs.append(r["out"])
        if valid.size == 0:
            assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t]))
        else:
            assert np.allclose(lse[t], r["lse"], atol=2e-3, rtol=1e-4), ("lse", t)
    assert swapped <= max(1, int(allow_swaps_frac * len(queries))), swapped
    e = np.stack(errs)
    rf = np.stack(refs)
    assert np.abs(e).max() <= 2e-2, float(np.abs(e).max())
    if np.linalg.norm(rf) > 0:
        assert np.linalg.norm(e) / np.linalg.norm(rf) <= 1e-2
    return swapped


@pytest.mark.parametrize("name", ["tiny", "tiny_seven", "tiny_padded_six", "tiny_batch", "mini_decode", "mini_decode_64",
                                  "mini_prefill", "mini_heavy"])
def test_chain_reduced(harness, name):
    wl = syn.get(name)
    say(f"chain {name} T={wl.T}")
    dw = harness.DeviceWorkload(wl, canary=0x11)
    dw.step()
    torch.cuda.synchronize()
    _check_chain(dw, range(wl.T))


def test_chain_twice_is_bitwise_identical(harness):
    wl = syn.mini_decode()
    say("chain determinism")
    dw = harness.DeviceWorkload(wl)
    dw.step()
    a = [x.clone() for x in (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)]
    dw.step()
    torch.cuda.synchronize()
    for x, y in zip(a, (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)):
        assert torch.equal(x, y)


FULL = ["decode_32k", "decode_262k_b8", "decode_1m_b4", "prefill_4k_on_131k"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_chain_full_size_sampled(harness, name):
    if os.environ.get("DSA_SKIP_FULL") == "1":
        pytest.skip("full-size workloads disabled by DSA_SKIP_FULL")
    wl = syn.get(name)
    say(f"chain full {name} T={wl.T} rows={wl.total_rows}")
    dw = harness.DeviceWorkload(wl)
    dw.step()
    torch.cuda.synchronize()
    if wl.T > 16:
        g = np.random.default_rng(99)
        queries = sorted(set([0, wl.T - 1] + list(g.choice(wl.T, size=6, replace=False))))
    else:
        queries = list(range(wl.T))
    say(f"chain full {name}: checking {len(queries)} queries on the CPU")
    _check_chain(dw, queries, pool_sample=64, allow_swaps_frac=0.25)
    if wl.T <= 64 and dw.stride <= 65536:
        # the launches the bench times (prepared calls; group lists are kept
        # for at most 64 queries and 65,536 pools) give the same bits
        say(f"chain full {name}: the timed launches")
        ref = [x.clone() for x in (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)]
        for x in (dw.pool_ids, dw.indices):
            x.fill_(0x5A5A5A5A)
        for x in (dw.scores, dw.out, dw.lse):
            x.fill_(float("nan"))
        dw.step_fast()
        torch.cuda.synchronize()
        for what, a, b in zip(("scores", "pool_ids", "indices", "out", "lse"), ref,
                              (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)):
            assert torch.equal(a, b), what
    del dw
    torch.cuda.empty_cache()


def test_prepared_calls_match_the_calls(harness):
    """The prepared (validated-once) calls give the same bits as the calls."""
    import torch
    wl = syn.get("mini_decode")
    dw = harness.DeviceWorkload(wl, replicas=2)
    say("prepared calls mini_decode")
    for r in range(2):
        dw.step(r)
        torch.cuda.synchronize()
        ref = [x.clone() for x in (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)]
        for x in (dw.pool_ids, dw.indices):
            x.fill_(0x5A5A5A5A)
        for x in (dw.scores, dw.out, dw.lse):
            x.fill_(float("nan"))
        dw.step_fast(r)
        dw.step_fast(r)                 # a second launch of the same prepared calls
        torch.cuda.synchronize()
        for name, a, b in zip(("scores", "pool_ids", "indices", "out", "lse"), ref,
                              (dw.scores, dw.pool_ids, dw.indices, dw.out, dw.lse)):
            assert torch.equal(a, b), (name, r)


@pytest.mark.parametrize("name,span", [("mini_decode", 3), ("mini_decode", 70), ("mini_decode_64", 5), ("mini_heavy", 5),
                                       ("mini_heavy", 130), ("decode_32k", 4)])
def test_append_scores_groups_matches_separate_calls(harness, name, span):
    """append_scores_groups gives the bytes of append_tokens then
    index_scores_groups (cache rows, pools, scores, group lists, and the
    selection made from them), with the pools the step completes poisoned
    beforehand: the single launch must rebuild them, not read them."""
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    if wl.T > 64:
        pytest.skip("group lists are kept for at most 64 queries")
    say(f"append_scores_groups {name} span={span}")
    dw = harness.DeviceWorkload(wl)
    d = wl.dims
    pb, pe = [], []
    for b in range(wl.B):
        f = int(wl.first_valid[b])
        nv = [(int(x) - f + 1) // d.kpool for x in wl.q_pos[wl.q_seq == b] if int(x) >= f]
        e = max(nv) if nv else 0
        pe.append(e)
        pb.append(max(e - span, 0))
    max_pools = max(e - s for s, e in zip(pb, pe))
    begin = torch.tensor(pb, dtype=torch.int32, device="cuda")
    end = torch.tensor(pe, dtype=torch.int32, device="cuda")
    pools0 = dw.pools[0].clone()
    for b in range(wl.B):
        base = int(wl.pool_base[b])
        pools0[base + pb[b]: base + pe[b]] = 7.0
    cache0 = dw.caches[0].clone()
    ws_bytes = dsa.lib().dsa_index_scores_select_workspace_bytes(ctypes.byref(dw.dims), wl.T, dw.stride)
    outs = []
    for fused in (False, True):
        pools, cache = pools0.clone(), cache0.clone()
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        scores = torch.full_like(dw.scores, float("nan"))
        idx = torch.full_like(dw.indices, 0x5A5A5A5A)
        pid = torch.full_like(dw.pool_ids, 0x5A5A5A5A)
        if fused:
            dsa.append_scores_groups(dw.dims, dw.latent_q, dw.slots_q, cache, dw.k, dw.gate, dw.ln_w, dw.ln_b,
                                     begin, end, max_pools, pools, dw.q_idx, dw.w, dw.seqs, dw.q_seq, dw.q_pos,
                                     scores, ws)
        else:
            dsa.append_tokens(dw.dims, dw.latent_q, dw.slots_q, cache, dw.k, dw.gate, dw.ln_w, dw.ln_b, dw.seqs,
                              begin, end, max_pools, pools)
            dsa.index_scores_groups(dw.dims, dw.q_idx, dw.w, pools, dw.seqs, dw.q_seq, dw.q_pos, scores, ws)
        dsa.topk_select_groups(dw.dims, scores, dw.seqs, dw.q_seq, dw.q_pos, idx, ws, pool_ids=pid)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (cache, pools.view(torch.int16), scores, ws, idx, pid)])
    # the separate calls rebuilt the poisoned pools exactly as the cache build did
    assert torch.equal(outs[0][1], dw.pools[0].view(torch.int16).cpu())
    for what, a, b in zip(("cache", "pools", "scores", "workspace", "indices", "pool_ids"), outs[0], outs[1]):
        assert torch.equal(a, b), what


@pytest.mark.parametrize("name,splits,case", [("mini_decode", 17, "lists"), ("mini_decode", 0, "lists"),
                                              ("mini_decode", 1, "lists"), ("mini_heavy", 17, "lists"),
                                              ("mini_heavy", 3, "lists"), ("decode_32k", 17, "lists"),
                                              ("decode_32k", 17, "equal_scores"), ("mini_decode", 17, "fp32_q"),
                                              ("mini_decode_64", 17, "lists")])
def test_topk_sparse_mla_matches_separate_calls(harness, name, splits, case):
    """topk_sparse_mla gives the bits of topk_select_groups then sparse_mla
    over its list: pool ids, index list, out and lse.  equal_scores (q_idx =
    0) fails every list check, so each workgroup takes the exact pass over the
    scores; fp32 q runs the two calls (no one-launch form)."""
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"topk_sparse_mla {name} splits={splits} {case}")
    dw = harness.DeviceWorkload(wl, num_splits=splits)
    if case == "equal_scores":
        dw.q_idx.zero_()
    q = dw.q.float() if case == "fp32_q" else dw.q
    dw.step_append()
    dw.step_scores_groups()
    outs = []
    for fused in (False, True):
        pid = torch.full_like(dw.pool_ids, 0x5A5A5A5A)
        idx = torch.full_like(dw.indices, 0x5A5A5A5A)
        out = torch.full_like(dw.out, float("nan"))
        lse = torch.full_like(dw.lse, float("nan"))
        if fused:
            dsa.topk_sparse_mla(dw.dims, dw.scores, dw.seqs, dw.q_seq, dw.q_pos, idx, dw._ws_ss(), q, dw.caches[0],
                                wl.scale, out, lse, splits, dw.ws_mla, pool_ids=pid)
        else:
            dsa.topk_select_groups(dw.dims, dw.scores, dw.seqs, dw.q_seq, dw.q_pos, idx, dw._ws_ss(), pool_ids=pid)
            dsa.sparse_mla(dw.dims, q, dw.caches[0], idx, wl.scale, out, lse, splits, dw.ws_mla)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (pid, idx, out, lse)])
    if case == "equal_scores":
        assert np.array_equal(outs[0][0][0].numpy(), np.arange(wl.dims.select_k))
    for what, a, b in zip(("pool_ids", "indices", "out", "lse"), outs[0], outs[1]):
        assert torch.equal(a, b), what


def test_timed_scoring_launch_gives_the_same_bits(harness):
    """A scoring launch that records its kernel events (the bench's timing
    hook) makes the bits of an ordinary one, and the events bracket it."""
    import sparse_attention_store_amd as dsa
    wl = syn.get("mini_decode")
    say("timed scoring launch mini_decode")
    dw = harness.DeviceWorkload(wl)
    dw.step_append_scores()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dw.scores, dw._ws_ss())]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    dw.scores.fill_(float("nan"))
    dsa.time_next_scoring_launch(a, b)
    dw.step_append_scores()
    torch.cuda.synchronize()
    assert a.elapsed_time(b) > 0.0
    assert torch.equal(ref[0], dw.scores) and torch.equal(ref[1], dw._ws_ss())
