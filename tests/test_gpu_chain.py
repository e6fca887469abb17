"""End-to-end parity of the whole path (GPU) against the oracle chain.

Decode workloads run exactly the launches the bench times
(dsa_harness.DeviceWorkload.step_fast: dsa_append_scores_groups, then
dsa_topk_sparse_mla) and are checked against the oracle query by query; the
general chain (DeviceWorkload.step) must then give the same bits.  Other
workloads (tiny geometry, prefill, more than 65,536 pools) run the general
chain.  oracle_chain.check_chain states the checks: pools and scores within
tolerance, pool ids and index lists bit-exact against the oracle's top-k and
expansion on the GPU's own scores, the top-k set against the fp64 chain up to
near-ties, cache rows bit-exact, and attention against the oracle on the
GPU's list.  No checked query is skipped.  Reduced-size workloads are checked
on every query; full-size ones on every decode query and on one seeded query
from each 64-query block of the prefill chunk (plus its first and last).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import dsa_synth as syn
from oracle_chain import check_chain

pytestmark = pytest.mark.gpu

OUTS = ("scores", "pool_ids", "indices", "out", "lse")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_harness
    return dsa_harness


def _snapshot(dw):
    return [getattr(dw, n).clone() for n in OUTS]


def _poison(dw):
    for x in (dw.pool_ids, dw.indices):
        x.fill_(0x5A5A5A5A)
    for x in (dw.scores, dw.out, dw.lse):
        x.fill_(float("nan"))


def _same_bits(dw, ref, what):
    for name, a in zip(OUTS, ref):
        assert torch.equal(a, getattr(dw, name)), (what, name)


def _run_and_check(dw, queries):
    """The bench's launches when they apply (then the general chain must give
    the same bits), else the general chain; then the oracle check."""
    fast = dw.fast_supported()
    say(f"  running {'the timed launches' if fast else 'the general chain'}")
    dw.step_fast() if fast else dw.step()
    torch.cuda.synchronize()
    rep = check_chain(dw, queries, say=say)
    say(f"  checked {rep['queries']} queries, {rep['near_tie_queries']} with near-tie set differences")
    if fast:
        ref = _snapshot(dw)
        _poison(dw)
        dw.step()
        torch.cuda.synchronize()
        _same_bits(dw, ref, "general chain vs timed launches")
    return rep


@pytest.mark.parametrize("name", ["tiny", "tiny_seven", "tiny_padded_six", "tiny_batch", "mini_decode", "mini_decode_64",
                                  "mini_prefill", "mini_heavy", "mini_long"])
def test_chain_reduced(harness, name):
    wl = syn.get(name)
    say(f"chain {name} T={wl.T}")
    dw = harness.DeviceWorkload(wl, canary=0x11)
    _run_and_check(dw, range(wl.T))


def test_chain_reduced_bf16_output(harness):
    """The bench's output dtype (bf16) on the timed launches."""
    wl = syn.get("mini_decode_64")
    say("chain mini_decode_64 bf16 out")
    dw = harness.DeviceWorkload(wl, out_dtype=torch.bfloat16)
    _run_and_check(dw, range(wl.T))


def test_chain_twice_is_bitwise_identical(harness):
    wl = syn.mini_decode()
    say("chain determinism")
    dw = harness.DeviceWorkload(wl)
    for step in (dw.step, dw.step_fast):
        step()
        a = _snapshot(dw)
        _poison(dw)
        step()
        torch.cuda.synchronize()
        _same_bits(dw, a, step.__name__)


FULL = ["decode_32k", "decode_262k_b8", "decode_1m_b4", "prefill_4k_on_131k"]
# the bench's output dtype for the decode configurations it times
FULL_OUT = {"decode_32k": torch.bfloat16, "decode_262k_b8": torch.bfloat16}


def _full_queries(wl):
    if wl.T <= 64:
        return list(range(wl.T))
    # one seeded query from each 64-query block (the prefill scoring kernel's
    # query blocks), plus the first and the last
    g = np.random.default_rng(99)
    return sorted(set([0, wl.T - 1] + [64 * j + int(g.integers(64)) for j in range(wl.T // 64)]))


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_chain_full_size(harness, name):
    if os.environ.get("DSA_SKIP_FULL") == "1":
        pytest.skip("full-size workloads disabled by DSA_SKIP_FULL")
    wl = syn.get(name)
    say(f"chain full {name} T={wl.T} rows={wl.total_rows}")
    dw = harness.DeviceWorkload(wl, out_dtype=FULL_OUT.get(name, torch.float32))
    queries = _full_queries(wl)
    say(f"chain full {name}: {len(queries)} queries checked on the CPU")
    _run_and_check(dw, queries)
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
                                       ("mini_heavy", 130), ("decode_32k", 4), ("mini_long", 6)])
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
                                              ("mini_decode_64", 17, "lists"), ("mini_long", 0, "lists"),
                                              ("mini_long", 17, "equal_scores"),
                                              pytest.param("decode_262k_b8", 0, "lists", marks=pytest.mark.slow),
                                              pytest.param("decode_262k_b8", 0, "equal_scores",
                                                           marks=pytest.mark.slow)])
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
        # every score 0: the lowest ids win (the tie rule), for every query with
        # more visible pools than the budget
        for t in range(wl.T):
            if wl.n_vis(t) > wl.dims.select_k:
                assert np.array_equal(outs[0][0][t].numpy(), np.arange(wl.dims.select_k)), t
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
