"""The INT8 pool cache (GPU) against the oracle's O2q / O3q.

* pool build: codes and scales bit-exact against the oracle's quantiser run on
  the GPU's own fp32 pool states (the kernel's check output), and against the
  oracle's fp64 pools up to rounding-boundary cases (oracle_chain.check_int8_pools);
* scores: against O3q on the GPU's own codes, rtol 1e-2 with a floor of 1e-2 x
  row RMS, -inf past the visible pools; the scoring pass with group lists
  gives the same bits as the plain one;
* the single launch (new tokens + scoring, completed pools poisoned
  beforehand) gives the bits of the separate calls;
* the whole decode step on INT8 pools (the bench's launches) against the
  oracle, stage by stage (oracle_chain.check_chain).
"""
import ctypes

import numpy as np
import pytest
import torch

import dsa_synth as syn
import oracle as O
from oracle_chain import check_chain, check_int8_pools, score_close

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_harness
    return dsa_harness


def _oracle_pools(wl, b):
    import sys, os
    from oracle_chain import OracleWorkload
    return OracleWorkload(wl).pools(b)


@pytest.mark.parametrize("name", ["tiny", "tiny_batch", "mini_decode", "mini_heavy"])
def test_index_pools_int8(harness, name):
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"index_pools_int8 {name}")
    dw = harness.DeviceWorkload(wl, pool_format="int8", build=False)
    d = wl.dims
    # k and gate of every position (the cache build's upload), then the pools
    dw.build_caches()
    npools = dw.pool_codes[0].shape[0]
    f32 = torch.full((npools, d.idx_dim), float("nan"), dtype=torch.float32, device="cuda")
    codes = torch.full_like(dw.pool_codes[0], 0x5A)
    scales = torch.full_like(dw.pool_scales[0], float("nan"))
    ends = [wl.n_pools(b) for b in range(wl.B)]
    dsa.index_pools_int8(dw.dims, dw.k, dw.gate, dw.ln_w, dw.ln_b, dw.seqs,
                         torch.zeros(wl.B, dtype=torch.int32, device="cuda"),
                         torch.tensor(ends, dtype=torch.int32, device="cuda"), max(ends), codes, scales, f32)
    torch.cuda.synchronize()
    c, s, x = codes.cpu().numpy(), scales.cpu().numpy(), f32.cpu().numpy()
    c0, s0 = dw.pool_codes[0].cpu().numpy(), dw.pool_scales[0].cpu().numpy()
    for b in range(wl.B):
        n = wl.n_pools(b)
        if n == 0:
            continue
        rows = slice(int(wl.pool_base[b]), int(wl.pool_base[b]) + n)
        # the build without the fp32 output wrote the same codes
        assert np.array_equal(c[rows], c0[rows]) and np.array_equal(s[rows], s0[rows]), b
        # stage-isolated: the quantiser on the GPU's own fp32 states, bit for bit
        oc, osc = O.quantize_pools(x[rows])
        assert np.array_equal(c[rows], oc) and np.array_equal(s[rows], osc), b
        # end-to-end: the oracle's fp64 pools
        check_int8_pools(c[rows], s[rows], _oracle_pools(wl, b), b)
        opools = _oracle_pools(wl, b)
        for p in range(n):
            ok, worst = score_close(x[rows][p], opools[p], d.idx_dim)
            assert ok, ("fp32 pool state", b, p, worst)


@pytest.mark.parametrize("name", ["mini_decode", "mini_decode_64", "mini_heavy", "decode_32k", "mini_long"])
def test_index_scores_int8(harness, name):
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"index_scores_int8 {name}")
    dw = harness.DeviceWorkload(wl, pool_format="int8")
    d = wl.dims
    dw.scores.fill_(float("nan"))
    dw.step_scores()
    torch.cuda.synchronize()
    sc = dw.scores.cpu().numpy()
    codes, scales = dw.pool_codes[0].cpu().numpy(), dw.pool_scales[0].cpu().numpy()
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        pb, n = int(wl.pool_base[b]), wl.n_pools(b)
        n_vis = wl.n_vis(t)
        ref = O.index_scores_int8(syn.gen_qidx(wl, t, t + 1)[0], syn.gen_w(wl, t, t + 1)[0], codes[pb:pb + n],
                                  scales[pb:pb + n], n_vis, dw.stride)
        ok, worst = score_close(sc[t], ref, n_vis)
        assert ok, (t, worst)
        assert np.all(np.isneginf(sc[t, n_vis:])), t
    # with group lists: the same scores, bit for bit
    ref = dw.scores.clone()
    dw.scores.fill_(float("nan"))
    dw.step_scores_groups()
    torch.cuda.synchronize()
    assert torch.equal(ref, dw.scores)


@pytest.mark.parametrize("name,span", [("mini_decode", 3), ("mini_decode", 70), ("mini_decode_64", 5),
                                       ("mini_heavy", 130), ("decode_32k", 4), ("mini_long", 6)])
def test_append_scores_groups_int8_matches_separate_calls(harness, name, span):
    """The single launch gives the bytes of store_int8 + index_pools_int8 +
    index_scores_groups_int8 (rows, codes, scales, scores, group lists, and
    the selection from them), with the pools the step completes poisoned
    beforehand: the launch must rebuild them, not read them."""
    import sparse_attention_store_amd as dsa
    wl = syn.get(name)
    say(f"append_scores_groups_int8 {name} span={span}")
    dw = harness.DeviceWorkload(wl, pool_format="int8")
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
    codes0, scales0 = dw.pool_codes[0].clone(), dw.pool_scales[0].clone()
    for b in range(wl.B):
        base = int(wl.pool_base[b])
        codes0[base + pb[b]: base + pe[b]] = 77
        scales0[base + pb[b]: base + pe[b]] = 3.0
    cache0 = dw.caches[0].clone()
    ws_bytes = dsa.lib().dsa_index_scores_select_workspace_bytes(ctypes.byref(dw.dims), wl.T, dw.stride)
    outs = []
    for fused in (False, True):
        codes, scales, cache = codes0.clone(), scales0.clone(), cache0.clone()
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        scores = torch.full_like(dw.scores, float("nan"))
        idx = torch.full_like(dw.indices, 0x5A5A5A5A)
        pid = torch.full_like(dw.pool_ids, 0x5A5A5A5A)
        if fused:
            dsa.append_scores_groups_int8(dw.dims, dw.latent_q, dw.slots_q, cache, dw.k, dw.gate, dw.ln_w, dw.ln_b,
                                          begin, end, max_pools, codes, scales, dw.q_idx, dw.w, dw.seqs, dw.q_seq,
                                          dw.q_pos, scores, ws)
        else:
            dsa.store_int8(dw.dims, dw.latent_q, dw.slots_q, cache)
            dsa.index_pools_int8(dw.dims, dw.k, dw.gate, dw.ln_w, dw.ln_b, dw.seqs, begin, end, max_pools, codes,
                                 scales)
            dsa.index_scores_groups_int8(dw.dims, dw.q_idx, dw.w, codes, scales, dw.seqs, dw.q_seq, dw.q_pos, scores,
                                         ws)
        dsa.topk_select_groups(dw.dims, scores, dw.seqs, dw.q_seq, dw.q_pos, idx, ws, pool_ids=pid)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (cache, codes, scales, scores, ws, idx, pid)])
    # the separate calls rebuilt the poisoned pools exactly as the cache build did
    assert torch.equal(outs[0][1], dw.pool_codes[0].cpu()) and torch.equal(outs[0][2], dw.pool_scales[0].cpu())
    for what, a, b in zip(("cache", "codes", "scales", "scores", "workspace", "indices", "pool_ids"), outs[0],
                          outs[1]):
        assert torch.equal(a, b), what


@pytest.mark.parametrize("name", ["mini_decode", "mini_decode_64", "mini_heavy", "mini_long",
                                  pytest.param("decode_32k", marks=pytest.mark.slow),
                                  pytest.param("decode_262k_b8", marks=pytest.mark.slow)])
def test_chain_int8(harness, name):
    """The bench's launches on INT8 pools, checked stage by stage; the general
    chain (separate calls) gives the same bits."""
    wl = syn.get(name)
    say(f"int8 chain {name}")
    out = torch.bfloat16 if name == "decode_262k_b8" else torch.float32
    dw = harness.DeviceWorkload(wl, pool_format="int8", out_dtype=out)
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
