"""The single-launch decode step (dsa_decode_step) on the GPU.

It must make, bit for bit, the selection of the separate calls it replaces
(scores -> topk_select_expand -> sparse_mla with one split per 128 list
positions), give their attention output up to the order of floating-point
sums (its workgroups have 4 waves, the separate kernel's 8, so per-row sums
are grouped differently), and match the oracle chain under the same rules as
tests/test_gpu_chain.py.  Its workspace control words must come back zero
(every call leaves the queue and the per-query counters reset), so a second
call gives the same bits, and no internal wait may time out.
"""
import numpy as np
import pytest
import torch

import dsa_synth as syn

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_harness
    return dsa_harness


def _same_attention(o_ref, lse_ref, o, lse):
    """out/lse equal up to the grouping of the per-row sums (a few fp32 ulps)."""
    o_ref, o = o_ref.float(), o.float()
    tol = 1e-5 * max(float(o_ref.abs().max()), 1.0)
    assert float((o - o_ref).abs().max()) <= tol, "out"
    fin = torch.isfinite(lse_ref)
    assert torch.equal(fin, torch.isfinite(lse)), "lse"
    if bool(fin.any()):
        assert float((lse[fin] - lse_ref[fin]).abs().max()) <= 1e-5, "lse"


def _fused_vs_separate(harness, wl, splits):
    import sparse_attention_store_amd as dsa
    dw = harness.DeviceWorkload(wl, num_splits=splits)
    dw.step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dw.pool_ids, dw.indices, dw.out, dw.lse)]
    for x in (dw.pool_ids, dw.indices):
        x.fill_(0x5A5A5A5A)
    dw.out.fill_(float("nan"))
    dw.lse.fill_(float("nan"))
    first = None
    for rep in range(2):
        dw.step_decode()
        torch.cuda.synchronize()
        assert dsa.decode_step_error(dw.ws_step) == 0
        ctl = dw.ws_step[:16].view(torch.int32).cpu().numpy()
        assert ctl[0] == 0 and ctl[1] == 0, ("queue not reset", ctl)
        for name, a, b in zip(("pool_ids", "indices"), ref, (dw.pool_ids, dw.indices)):
            assert torch.equal(a, b), (name, rep)
        _same_attention(ref[2], ref[3], dw.out, dw.lse)
        cur = [x.clone() for x in (dw.out, dw.lse)]
        if first is None:
            first = cur
        else:                                          # run to run: bit for bit
            assert all(torch.equal(a, b) for a, b in zip(first, cur))
    return dw


@pytest.mark.parametrize("name", ["mini_decode", "mini_heavy"])
def test_decode_step_matches_separate_calls(harness, name):
    wl = syn.get(name)
    say(f"decode step {name} T={wl.T} H={wl.dims.mla_heads}")
    _fused_vs_separate(harness, wl, splits=17)


def test_decode_step_matches_oracle(harness):
    from oracle_chain import check_chain
    import sparse_attention_store_amd as dsa
    wl = syn.mini_decode()
    say(f"decode step vs oracle {wl.name}")
    dw = harness.DeviceWorkload(wl, num_splits=17)
    dw.step()                                   # fills dw.scores (checked by the chain rules)
    dw.step_decode()
    torch.cuda.synchronize()
    assert dsa.decode_step_error(dw.ws_step) == 0
    check_chain(dw, range(wl.T), say=say)


def test_decode_step_forced_fallback(harness):
    """Equal scores everywhere (q_idx = 0): every kept-group list is full and
    every certificate fails, so each sparse query takes the exact streaming
    select over its scores; the result must still be the lowest ids."""
    import sparse_attention_store_amd as dsa
    wl = syn.decode_32k()
    say("decode step with all-equal scores (fallback path)")
    dw = harness.DeviceWorkload(wl, num_splits=17)
    dw.q_idx.zero_()
    dw.step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dw.pool_ids, dw.indices, dw.out, dw.lse)]
    dw.step_decode()
    torch.cuda.synchronize()
    assert dsa.decode_step_error(dw.ws_step) == 0
    sk = wl.dims.select_k
    assert np.array_equal(dw.pool_ids[0].cpu().numpy(), np.arange(sk))
    for a, b in zip(ref, (dw.pool_ids, dw.indices)):
        assert torch.equal(a, b)
    _same_attention(ref[2], ref[3], dw.out, dw.lse)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode_32k", "decode_262k_b8"])
def test_decode_step_full_size(harness, name):
    from oracle_chain import check_chain
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"decode step full {name} T={wl.T}")
    dw = _fused_vs_separate(harness, wl, splits=17)
    assert dsa.decode_step_error(dw.ws_step) == 0
    say(f"decode step full {name}: oracle check of {wl.T} queries")
    check_chain(dw, list(range(wl.T)), say=say)
    del dw
    torch.cuda.empty_cache()
