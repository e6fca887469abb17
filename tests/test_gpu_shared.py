"""Runs of queries that share one pass over their sequence's pools
(dsa_append_scores_groups_shared): the same bits as the one-query launch
(cache rows, pools, scores, group lists, the selection made from them), with
the pools the step completes poisoned beforehand, for bf16 and INT8 pools and
runs of 2 and 4; then the whole decode step on a 4-queries-per-sequence batch
against the oracle, stage by stage.

mini_decode and mini_decode_64 give runs whose queries sit at scattered
positions (very different visible counts, one inside the padding);
mini_mtp and decode_262k_b8_mtp give the speculative-decode layout (each
sequence's last 4 positions)."""
import ctypes

import numpy as np
import pytest
import torch

import dsa_synth as syn
from oracle_chain import check_chain

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_harness
    return dsa_harness


CASES = [("mini_mtp", "bf16", 4), ("mini_mtp", "int8", 4), ("mini_mtp", "bf16", 2), ("mini_decode", "bf16", 4),
         ("mini_decode", "int8", 3), ("mini_decode_64", "bf16", 4), ("mini_decode_64", "int8", 4),
         pytest.param("decode_262k_b8_mtp", "bf16", 4, marks=pytest.mark.slow),
         pytest.param("decode_262k_b8_mtp", "int8", 4, marks=pytest.mark.slow)]


@pytest.mark.parametrize("name,pools,share", CASES)
def test_shared_matches_one_query_launch(harness, name, pools, share):
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"shared runs {name} {pools} share={share}")
    dw = harness.DeviceWorkload(wl, pool_format=pools)
    d = wl.dims
    int8 = pools == "int8"
    pool_bufs = (dw.pool_codes[0], dw.pool_scales[0]) if int8 else (dw.pools[0],)
    ref_pools = [x.clone() for x in pool_bufs]
    # poison the pools this step completes: both launches must rebuild them
    poisoned = [x.clone() for x in pool_bufs]
    for b in range(wl.B):
        base = int(wl.pool_base[b])
        s0, e0 = int(dw.step_pool_begin[b]), int(dw.step_pool_end[b])
        for x in poisoned:
            x[base + s0: base + e0] = 7
    cache0 = dw.caches[0].clone()
    ws_bytes = dsa.lib().dsa_index_scores_select_workspace_bytes(ctypes.byref(dw.dims), wl.T, dw.stride)
    outs = []
    for shared in (False, True):
        pb = [x.clone() for x in poisoned]
        cache = cache0.clone()
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        scores = torch.full_like(dw.scores, float("nan"))
        idx = torch.full_like(dw.indices, 0x5A5A5A5A)
        pid = torch.full_like(dw.pool_ids, 0x5A5A5A5A)
        args = (dw.dims, dw.latent_q, dw.slots_q, cache, dw.k, dw.gate, dw.ln_w, dw.ln_b, dw.step_pool_begin,
                dw.step_pool_end, dw.step_max_pools)
        tail = (dw.q_idx, dw.w, dw.seqs, dw.q_seq, dw.q_pos, scores, ws)
        if shared:
            dsa.append_scores_groups_shared(*args, pb[0], pb[1] if int8 else None, *tail, share)
        elif int8:
            dsa.append_scores_groups_int8(*args, pb[0], pb[1], *tail)
        else:
            dsa.append_scores_groups(*args, pb[0], *tail)
        dsa.topk_select_groups(dw.dims, scores, dw.seqs, dw.q_seq, dw.q_pos, idx, ws, pool_ids=pid)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in [cache] + pb + [scores, ws, idx, pid]])
    # both rebuilt the poisoned pools exactly as the cache build did
    for a, r in zip(outs[1][1:1 + len(ref_pools)], ref_pools):
        assert torch.equal(a, r.cpu())
    names = ["cache"] + ["pools"] * len(ref_pools) + ["scores", "workspace", "indices", "pool_ids"]
    for what, a, b in zip(names, outs[0], outs[1]):
        assert torch.equal(a, b), what


@pytest.mark.parametrize("name,pools", [("mini_mtp", "bf16"), ("mini_mtp", "int8"),
                                        pytest.param("decode_262k_b8_mtp", "bf16", marks=pytest.mark.slow)])
def test_chain_shared(harness, name, pools):
    """A speculative decode step through the timed launches with shared runs,
    checked stage by stage; the general chain gives the same bits."""
    wl = syn.get(name)
    say(f"shared chain {name} {pools}")
    out = torch.bfloat16 if name == "decode_262k_b8_mtp" else torch.float32
    dw = harness.DeviceWorkload(wl, pool_format=pools, share=4, out_dtype=out)
    assert dw.fast_supported()
    dw.step_fast()
    torch.cuda.synchronize()
    rep = check_chain(dw, range(wl.T), say=say)
    say(f"  {rep}")
    names = ("scores", "pool_ids", "indices", "out", "lse")
    ref = [getattr(dw, n).clone() for n in names]
    dw.step()
    torch.cuda.synchronize()
    for n, a in zip(names, ref):
        assert torch.equal(a, getattr(dw, n)), n
