"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test pins one function against what the pages state, a closed form, a
special case that reduces to a textbook routine (torch CPU ops in float64), a
hand-worked fixture under tests/golden/, or brute force on tiny inputs.
"""
import heapq
import os

import numpy as np
import pytest
import torch

import dsa_synth as syn
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ O1 INT8 row

def test_store_int8_worked_row_half_even():
    x = np.zeros((1, 64), dtype=np.float32)
    expect = np.zeros(64, dtype=np.int8)
    scale_bytes = None
    for ln in _golden_lines("store_int8_halfeven.txt"):
        parts = ln.split()
        if parts[0] == "scale_bytes":
            scale_bytes = bytes(int(v, 16) for v in parts[1:])
            continue
        i, v, c = int(parts[0]), float(parts[1]), int(parts[2])
        x[0, i] = v
        expect[i] = c
    cache = np.full((3, 80), 0xAB, dtype=np.uint8)
    O.store_int8(x, np.array([1]), cache)
    row = cache[1]
    assert np.array_equal(row[:64].view(np.int8), expect)
    assert bytes(row[64:68]) == scale_bytes
    assert np.all(row[68:] == 0)
    assert np.all(cache[0] == 0xAB) and np.all(cache[2] == 0xAB)


def test_store_int8_row_layout_528():
    assert O.row_bytes_for(512) == 528 and O.row_bytes_for(64) == 80
    g = np.random.default_rng(0)
    x = syn.bf16_round(g.standard_normal((5, 512)).astype(np.float32))
    cache = np.zeros((5, 528), dtype=np.uint8)
    O.store_int8(x, np.arange(5), cache)
    scales = cache[:, 512:516].copy().view("<f4")[:, 0]
    assert np.all(cache[:, 516:] == 0)                       # 12 zero bytes
    assert np.allclose(scales, np.abs(x).max(axis=1) / 127.0, rtol=1e-6)


def test_store_int8_invariants_random_rows():
    g = np.random.default_rng(1)
    x = (g.standard_t(3, size=(400, 512)) * g.uniform(1e-3, 50, size=(400, 1))).astype(np.float32)
    codes, s = O.quantize_rows(x)
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 2.0 ** -15))
    amax_col = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(400), amax_col]
    assert np.all(np.abs(top.astype(int)) == 127)
    assert codes.min() >= -127


def test_store_int8_constant_and_zero_rows():
    x = np.zeros((3, 64), dtype=np.float32)
    x[0] = 2.5
    x[1] = -0.75
    codes, s = O.quantize_rows(x)
    assert np.all(codes[0] == 127) and np.all(codes[1] == -127)
    assert s[0] == np.float32(2.5) / np.float32(127) and s[1] == np.float32(0.75) / np.float32(127)
    assert np.all(codes[2] == 0) and np.isfinite(s[2]) and s[2] > 0   # floored, no division by zero


def test_store_int8_skips_negative_slots():
    x = np.ones((3, 64), dtype=np.float32)
    cache = np.full((4, 80), 7, dtype=np.uint8)
    O.store_int8(x, np.array([-1, 2, -5]), cache)
    assert np.all(cache[[0, 1, 3]] == 7) and not np.all(cache[2] == 7)


# ------------------------------------------------------------------ O2 pools

# ------------------------------------------------------------------ O1 read back: dequantize_rows

def _row_bytes_by_hand(codes, scale, row_bytes, pad_byte=0):
    """One stored row assembled with struct, independently of pack_rows: the
    codes as two's-complement bytes, the scale as a little-endian IEEE float,
    then pad bytes ([GLM-5.3 Kernels, Included]: codes, one fp32 scale, padding)."""
    import struct
    body = struct.pack("<%db" % len(codes), *codes) + struct.pack("<f", scale)
    return np.frombuffer(body + bytes([pad_byte]) * (row_bytes - len(body)), dtype=np.uint8)


def _dequant_pins_hold(fn):
    """The facts a correct read-back of the row layout must reproduce; returns
    the first one that fails (None when all hold)."""
    # (a) hand-built rows: negative codes read as negative, the scale read from
    # bytes D .. D+4 (pad bytes are not the scale), exact products
    codes = [-127, -1, 0, 1, 2, 127, -2, -64] + [5] * 56
    rows = np.stack([_row_bytes_by_hand(codes, 0.5, 80, pad_byte=0x3F),
                     _row_bytes_by_hand(codes[::-1], 2.0 ** -7, 80, pad_byte=0x41)])
    got = fn(rows, 64)
    want = np.stack([np.array(codes, np.float64) * 0.5, np.array(codes[::-1], np.float64) * 2.0 ** -7])
    if got.shape != want.shape or not np.array_equal(got, want):
        return "hand-built rows"
    # (b) round trip through the stored bytes: within s/2 of the source, signs kept
    g = np.random.default_rng(5)
    x = (g.standard_t(3, size=(64, 512)) * g.uniform(1e-3, 40, size=(64, 1))).astype(np.float32)
    cache = np.zeros((64, 528), dtype=np.uint8)
    O.store_int8(x, np.arange(64), cache)
    deq = fn(cache, 512)
    s = np.abs(x).max(axis=1).astype(np.float64) / 127.0
    if not np.all(np.abs(deq - x) <= s[:, None] / 2 * (1 + 2.0 ** -15)):
        return "round trip error above s/2"
    if not np.all((np.sign(deq) == np.sign(x)) | (deq == 0)):
        return "sign flipped"
    return None


def test_dequantize_rows_reads_the_stored_layout():
    assert _dequant_pins_hold(O.dequantize_rows) is None


def test_dequantize_pins_reject_plausible_mistakes():
    """Mistakes planted in copies of the read-back (on the CPU): codes read as
    uint8, the scale taken from the pad bytes, the scale read big-endian."""
    def as_uint8(rows, d):
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        return rows[:, :d].astype(np.float64) * rows[:, d:d + 4].copy().view("<f4").astype(np.float64)

    def scale_from_pad(rows, d):
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        return rows[:, :d].view(np.int8).astype(np.float64) * rows[:, d + 4:d + 8].copy().view("<f4").astype(np.float64)

    def big_endian(rows, d):
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        return rows[:, :d].view(np.int8).astype(np.float64) * rows[:, d:d + 4].copy().view(">f4").astype(np.float64)

    for bad in (as_uint8, scale_from_pad, big_endian):
        assert _dequant_pins_hold(bad) is not None, bad.__name__


def _torch_pools(k_rows, gate_rows, w, b, eps):
    """Textbook reference for one pool: torch layer_norm, softmax over the 4 slots."""
    k = torch.tensor(k_rows, dtype=torch.float64)
    gt = torch.tensor(gate_rows, dtype=torch.float64)
    y = torch.nn.functional.layer_norm(k, (k.shape[-1],), torch.tensor(w, dtype=torch.float64),
                                       torch.tensor(b, dtype=torch.float64), eps)
    a = torch.softmax(gt, dim=0)
    return (a * y).sum(0).numpy()


def test_seven_tokens_make_one_pool():
    wl = syn.tiny_seven()
    k, g = syn.gen_kgate(wl, 0, 0, 7)
    lw, lb = syn.gen_ln(wl)
    pools = O.pool_states(k, g, lw, lb, 1e-5, 0, 7, 4)
    assert pools.shape == (1, 32)
    assert np.allclose(pools[0], _torch_pools(k[0:4], g[0:4], lw, lb, 1e-5), rtol=1e-12, atol=1e-12)


def test_left_padding_pool_starts_at_first_valid():
    wl = syn.tiny_padded_six()                 # [P, P, A, B, C, D]
    k, g = syn.gen_kgate(wl, 0, 0, 6)
    assert np.all(np.abs(k[:2]) == syn.POISON)  # padding carries poison
    lw, lb = syn.gen_ln(wl)
    pools = O.pool_states(k, g, lw, lb, 1e-5, 2, 6, 4)
    assert pools.shape == (1, 32)
    assert np.allclose(pools[0], _torch_pools(k[2:6], g[2:6], lw, lb, 1e-5), rtol=1e-12, atol=1e-12)
    wrong = _torch_pools(k[0:4], g[0:4], lw, lb, 1e-5)    # a pool anchored at slot 0
    assert not np.allclose(pools[0], wrong, atol=1e-3)


def test_pools_match_textbook_layernorm_and_slot_softmax():
    wl = syn.tiny()
    k, g = syn.gen_kgate(wl, 0, 0, 64)
    lw, lb = syn.gen_ln(wl)
    pools = O.pool_states(k, g, lw, lb, 1e-5, 5, 64, 4)
    assert pools.shape == (14, 32)
    for p in range(14):
        t0 = 5 + 4 * p
        ref = _torch_pools(k[t0:t0 + 4], g[t0:t0 + 4], lw, lb, 1e-5)
        assert np.allclose(pools[p], ref, rtol=1e-12, atol=1e-12)


def test_slot_weights_sum_to_one_per_channel():
    g = np.random.default_rng(2)
    k = g.standard_normal((40, 128))
    gate = g.standard_normal((40, 128)) * 3
    _, a = O.pool_states(k, gate, np.ones(128), np.zeros(128), 1e-5, 3, 40, 4, return_weights=True)
    assert a.shape == (9, 4, 128)
    assert np.allclose(a.sum(axis=1), 1.0, atol=1e-14)
    assert not np.allclose(a.sum(axis=2), 1.0)          # not a softmax over channels


def test_layernorm_bias_is_applied():
    g = np.random.default_rng(3)
    k = g.standard_normal((12, 32))
    gate = g.standard_normal((12, 32))
    ln_b = g.standard_normal(32)
    pools = O.pool_states(k, gate, np.zeros(32), ln_b, 1e-5, 0, 12, 4)
    assert np.allclose(pools, ln_b[None, :], rtol=0, atol=1e-14)


def test_equal_gates_average_and_dominant_gate_selects():
    g = np.random.default_rng(4)
    k = g.standard_normal((4, 32))
    lw, lb = g.standard_normal(32), g.standard_normal(32)
    ln = torch.nn.functional.layer_norm(torch.tensor(k), (32,), torch.tensor(lw), torch.tensor(lb), 1e-5).numpy()
    pools = O.pool_states(k, np.zeros((4, 32)), lw, lb, 1e-5, 0, 4, 4)
    assert np.allclose(pools[0], ln.mean(axis=0), atol=1e-13)
    gate = np.full((4, 32), -200.0)
    gate[2] = 200.0
    pools = O.pool_states(k, gate, lw, lb, 1e-5, 0, 4, 4)
    assert np.allclose(pools[0], ln[2], atol=1e-12)


def test_layer_norm_is_normalising_with_unit_affine():
    g = np.random.default_rng(5)
    x = g.standard_normal((50, 128)) * 7 + 3
    y = O.layer_norm(x, np.ones(128), np.zeros(128), 0.0)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, atol=1e-12)


def test_store_bf16_ties_to_even_and_library_agreement():
    one = 1.0
    assert O.store_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                 # tie -> even (mantissa 0)
    assert O.store_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even (mantissa 2)
    assert O.store_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert O.store_bf16(np.array([-3.0, 0.0, 96.0]))[0:3].tolist() == [-3.0, 0.0, 96.0]
    g = np.random.default_rng(14)
    x = (g.standard_normal(20000) * 10.0 ** g.uniform(-3, 3, 20000)).astype(np.float32).astype(np.float64)
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.store_bf16(x), ref)
    assert np.all(np.abs(O.store_bf16(x) - x) <= np.abs(x) * 2.0 ** -8)


# ------------------------------------------------------------------ O3 scores

def test_scores_single_head_unit_weight_is_relu_dot():
    g = np.random.default_rng(6)
    q = g.standard_normal((1, 128))
    pools = g.standard_normal((30, 128))
    s = O.index_scores(q, np.array([1.0]), pools, 30)
    assert np.allclose(s, np.maximum(pools @ q[0], 0.0), atol=1e-12)


def test_scores_unit_vector_queries_pick_channels():
    g = np.random.default_rng(7)
    pools = g.standard_normal((20, 128))
    q = np.zeros((32, 128))
    q[5, 17] = 1.0
    q[9, 3] = 1.0
    w = np.zeros(32)
    w[5], w[9] = 2.0, -0.5
    s = O.index_scores(q, w, pools, 20)
    assert np.allclose(s, 2.0 * np.maximum(pools[:, 17], 0) - 0.5 * np.maximum(pools[:, 3], 0), atol=1e-12)


def test_scores_zero_query_and_invisible_tail():
    pools = np.random.default_rng(8).standard_normal((10, 32))
    s = O.index_scores(np.zeros((4, 32)), np.ones(4), pools, 6, stride=10)
    assert np.all(s[:6] == 0.0) and np.all(np.isneginf(s[6:]))


def test_scores_linear_in_weights_homogeneous_in_query():
    g = np.random.default_rng(9)
    q, pools = g.standard_normal((32, 128)), g.standard_normal((50, 128))
    w1, w2 = g.random(32), g.standard_normal(32)
    s = lambda qq, ww: O.index_scores(qq, ww, pools, 50)
    assert np.allclose(s(q, w1 + w2), s(q, w1) + s(q, w2), atol=1e-10)
    assert np.allclose(s(2.5 * q, w1), 2.5 * s(q, w1), atol=1e-10)
    assert not np.allclose(s(-q, w1), -s(q, w1))         # ReLU is applied per head


# ------------------------------------------------------------------ O4 top-k

def test_topk_hand_worked_ties():
    for ln in _golden_lines("topk_ties.txt"):
        k, sc, ex = [p.split() for p in ln.split("|")]
        scores = np.array([float(v) for v in sc])
        ids = O.topk_pools(scores, len(scores), int(k[0]))
        assert ids.tolist() == [int(v) for v in ex], ln


def test_topk_brute_force_and_invariants():
    g = np.random.default_rng(10)
    for trial in range(60):
        n = int(g.integers(1, 300))
        sel_k = int(g.integers(1, 40))
        scores = np.round(g.standard_normal(n) * 3, 1)            # many ties
        ids = O.topk_pools(scores, n, sel_k)
        kk = min(sel_k, n)
        brute = sorted(i for _, i in heapq.nsmallest(kk, [(-s, i) for i, s in enumerate(scores)]))
        assert ids[:kk].tolist() == brute
        assert np.all(ids[kk:] == -1)
        chosen = np.zeros(n, dtype=bool)
        chosen[ids[:kk]] = True
        if kk < n:
            assert scores[chosen].min() >= scores[~chosen].max()
        assert np.all(np.diff(ids[:kk]) > 0)


def test_topk_all_equal_picks_lowest_ids_and_dense_regime():
    assert O.topk_pools(np.zeros(1000), 1000, 512).tolist() == list(range(512))
    assert O.topk_pools(np.zeros(0), 0, 4).tolist() == [-1] * 4
    r = O.topk_pools(np.array([3.0, -1.0, 2.0]), 3, 4)
    assert r.tolist() == [0, 1, 2, -1]


# ------------------------------------------------------------------ O5 expansion

def test_expand_worked_counts():
    for ln in _golden_lines("expand_counts.txt"):
        a, nv, nvalid, ninv = [p.split() for p in ln.split("|")]
        f, sl, q = (int(v) for v in a)
        n_vis = O.visible_pool_count(q, f, 4)
        assert n_vis == int(nv[0]), ln
        ids = O.topk_pools(np.zeros(max(n_vis, 1)), n_vis, 4)
        out = O.expand_selection(ids, f, q, 100, 4, 24)
        assert out.shape == (24,)
        assert int((out >= 0).sum()) == int(nvalid[0]) and int((out == -1).sum()) == int(ninv[0]), ln
        v = out[out >= 0]
        assert np.all(np.diff(v) > 0)
        assert np.all(O.visible(q, f, v - 100))


def test_expand_dense_regime_is_every_visible_position():
    for f, q in [(5, 23), (0, 6), (3, 100), (2, 9)]:
        n_vis = O.visible_pool_count(q, f, 4)
        sel_k = 32
        ids = O.topk_pools(np.ones(max(n_vis, 1)), n_vis, sel_k)
        out = O.expand_selection(ids, f, q, 1000, 4, 4 * sel_k + 3)
        assert out[out >= 0].tolist() == [1000 + x for x in range(f, q + 1)]


def test_expand_production_width_full_budget():
    ids = np.arange(0, 1024, 2, dtype=np.int32)          # 512 pools
    out = O.expand_selection(ids, 3, 3 + 4 * 600 + 2, 0, 4, 2176)
    assert int((out >= 0).sum()) == 2048 + 3 and np.all(out[2051:] == -1)


# ------------------------------------------------------------------ O6/O7 attention

def _cache_from(latent):
    cache = np.zeros((latent.shape[0], O.row_bytes_for(latent.shape[1])), dtype=np.uint8)
    O.store_int8(latent, np.arange(latent.shape[0]), cache)
    return cache


def test_attention_single_row_identical_rows_and_zero_scale():
    g = np.random.default_rng(11)
    lat = g.standard_normal((40, 64)).astype(np.float32)
    cache = _cache_from(lat)
    deq = O.dequantize_rows(cache, 64)
    q = g.standard_normal((3, 64))
    idx = np.full(24, -1)
    idx[7] = 13
    o, lse = O.sparse_mla(q, cache, idx, 0.125, 64)
    assert np.allclose(o, deq[13][None, :], atol=1e-14)
    assert np.allclose(lse, 0.125 * q @ deq[13], atol=1e-12)
    same = np.repeat(lat[:1], 40, axis=0)
    o, _ = O.sparse_mla(q, _cache_from(same), np.arange(24), 0.5, 64)
    assert np.allclose(o, O.dequantize_rows(_cache_from(same[:1]), 64)[0][None, :], atol=1e-13)
    sel = np.array([1, 5, 9, 30, -1, -1])
    o, _ = O.sparse_mla(q, cache, sel, 0.0, 64)
    assert np.allclose(o, deq[[1, 5, 9, 30]].mean(axis=0)[None, :], atol=1e-13)


def test_attention_empty_list_and_permutation_invariance():
    g = np.random.default_rng(12)
    lat = g.standard_normal((50, 64)).astype(np.float32)
    cache = _cache_from(lat)
    q = g.standard_normal((2, 64))
    o, lse = O.sparse_mla(q, cache, np.full(24, -1), 0.125, 64)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    idx = np.array([3, 8, 20, 41, -1, 7, -1, -1])
    o1, l1 = O.sparse_mla(q, cache, idx, 0.125, 64)
    o2, l2 = O.sparse_mla(q, cache, idx[::-1].copy(), 0.125, 64)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_attention_equals_brute_force_masked_dense_on_tiny():
    """Whole tiny chain: the list-based attention equals dense attention with the mask."""
    wl = syn.tiny()
    d = wl.dims
    k, g = syn.gen_kgate(wl, 0, 0, 64)
    lw, lb = syn.gen_ln(wl)
    lat = syn.gen_latent(wl, 0, 0, 64)
    cache = _cache_from(lat)
    keys = O.dequantize_rows(cache, d.latent_dim)
    pools = O.pool_states(k, g, lw, lb, d.ln_eps, 5, 64, 4)
    qi, w, q = syn.gen_qidx(wl, 0, 64), syn.gen_w(wl, 0, 64), syn.gen_q(wl, 0, 64)
    for t in range(64):
        n_vis = O.visible_pool_count(t, 5, 4)
        sc = O.index_scores(qi[t], w[t], pools, n_vis)
        ids = O.topk_pools(sc, n_vis, d.select_k)
        idx = O.expand_selection(ids, 5, t, 0, 4, d.out_width)
        o, lse = O.sparse_mla(q[t], cache, idx, wl.scale, d.latent_dim)
        mask = O.topk_to_mask(idx, 0, 64) & O.visible(t, 5, np.arange(64))
        ob, lb_ = O.masked_attention(q[t], keys, mask, wl.scale)
        assert np.allclose(o, ob, atol=1e-12)
        if t < 5:
            assert np.all(idx == -1) and np.all(o == 0)


def test_dense_regime_equals_textbook_causal_attention():
    """With no more visible pools than the budget, DSA is causal attention over [f, q]."""
    wl = syn.tiny()
    lat = syn.gen_latent(wl, 0, 0, 64)
    cache = _cache_from(lat)
    keys = torch.tensor(O.dequantize_rows(cache, 64))
    q = syn.gen_q(wl, 0, 64)
    f = 5
    for t in range(f, 24):                      # n_vis <= 4 = select_k
        n_vis = O.visible_pool_count(t, f, 4)
        ids = O.topk_pools(np.ones(max(n_vis, 1)), n_vis, 4)
        idx = O.expand_selection(ids, f, t, 0, 4, 24)
        o, _ = O.sparse_mla(q[t], cache, idx, wl.scale, 64)
        kv = keys[f:t + 1][None]                # [1, n, D]
        qt = torch.tensor(q[t], dtype=torch.float64)[:, None, :]     # [H, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kv.expand(2, -1, -1), kv.expand(2, -1, -1), scale=wl.scale)[:, 0, :].numpy()
        assert np.allclose(o, ref, atol=1e-12)


def test_generator_blocks_are_reproducible_and_bf16_exact():
    wl = syn.mini_decode()
    a = syn.gen_latent(wl, 1, 4000, 4200)
    b = syn.gen_latent(wl, 1, 4090, 4100)
    assert np.array_equal(a[90:100], b)
    assert np.array_equal(syn.bf16_round(a), a)
    k, _ = syn.gen_kgate(wl, 2, 0, 8)
    assert np.all(np.abs(k[:3]) == syn.POISON) and not np.any(np.abs(k[3:]) == syn.POISON)


# ------------------------------------------------------------------ O2q/O3q INT8 pool cache

def test_pool_int8_worked_row_and_score():
    vals, codes, score = [], [], None
    for ln in _golden_lines("pool_int8_worked.txt"):
        parts = ln.split()
        if parts[0] == "score":
            score = float(parts[1])
            continue
        vals.append(float(parts[1]))
        codes.append(int(parts[2]))
    pool = np.array([vals], dtype=np.float64)
    c, s = O.quantize_pools(pool)
    assert np.array_equal(c[0], np.array(codes, dtype=np.int8))
    assert s[0] == np.float32(1.0)
    q = np.zeros((2, 8))
    q[0, 0], q[0, 1] = 1.0, -1.0
    q[1, 0], q[1, 1] = 1.0, 2.0
    got = O.index_scores_int8(q, np.array([1.0, 0.5]), c, s, 1)
    assert got[0] == score


def test_int8_scores_equal_exact_scores_when_pools_are_on_the_grid():
    """Pools whose values are integers times 2^-3 with amax 127 * 2^-3 quantise
    without error (scale 2^-3 exactly), so the INT8 scores are O3's."""
    g = np.random.default_rng(21)
    codes = g.integers(-127, 128, size=(300, 128))
    codes[:, 5] = 127
    pools = codes * 2.0 ** -3
    c, s = O.quantize_pools(pools)
    assert np.all(s == np.float32(2.0 ** -3)) and np.array_equal(c.astype(np.int64), codes)
    qi = g.standard_normal((32, 128))
    w = g.random(32)
    assert np.array_equal(O.index_scores_int8(qi, w, c, s, 300, 320), O.index_scores(qi, w, pools, 300, 320))


def test_int8_scores_are_homogeneous_in_the_pool_scale():
    """Scaling a pool by a power of two leaves its codes unchanged and scales
    its scale, so its INT8 score scales by exactly that power of two."""
    g = np.random.default_rng(22)
    pools = g.standard_normal((64, 128)) * 3
    qi = g.standard_normal((32, 128))
    w = g.random(32)
    c1, s1 = O.quantize_pools(pools)
    c2, s2 = O.quantize_pools(pools * 8.0)
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(8.0))
    a = O.index_scores_int8(qi, w, c1, s1, 64)
    b = O.index_scores_int8(qi, w, c2, s2, 64)
    assert np.allclose(b, 8.0 * a, rtol=1e-14, atol=0)


def test_int8_pool_round_trip_within_half_a_step():
    g = np.random.default_rng(23)
    pools = g.standard_t(3, size=(500, 128)) * g.uniform(1e-3, 30, size=(500, 1))
    c, s = O.quantize_pools(pools)
    x32 = pools.astype(np.float32).astype(np.float64)
    err = np.abs(O.dequantize_pools(c, s) - x32)
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 2.0 ** -15))
    assert np.all(np.abs(c[np.arange(500), np.argmax(np.abs(pools), axis=1)].astype(int)) == 127)


def test_accuracy_figures_closed_forms():
    g = np.random.default_rng(24)
    r = g.standard_normal((4, 64))
    assert O.int8_accuracy(r, r) == (0.0, pytest.approx(1.0, abs=1e-15))
    nmse, cos = O.int8_accuracy(2 * r, r)
    assert nmse == pytest.approx(1.0, rel=1e-12) and cos == pytest.approx(1.0, abs=1e-12)
    a = np.zeros(8); a[0] = 1
    b = np.zeros(8); b[1] = 1
    assert O.int8_accuracy(a, b) == (pytest.approx(2.0), pytest.approx(0.0))


def test_int8_mla_accuracy_against_bf16_latents():
    """The accuracy figures of INT8 MLA against attention over the source bf16
    latents on the same list (reported, not gated): decode_32k's query on its
    oracle list, and the heavy-tailed mini_heavy queries.  The loose bounds
    below only catch a broken quantiser."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from oracle_chain import OracleWorkload
    rep = []
    for name in ("decode_32k", "mini_heavy"):
        wl = syn.get(name)
        ow = OracleWorkload(wl)
        for t in range(wl.T):
            r = ow.query(t)
            b = int(wl.q_seq[t])
            valid = r["indices"][r["indices"] >= 0] - int(wl.row_base[b])
            if valid.size == 0:
                continue
            blk = syn.ROW_BLOCK
            lat = np.stack([ow._latent_block(b, int(x) // blk)[int(x) % blk] for x in valid])
            q = syn.gen_q(wl, t, t + 1)[0]
            o_ref = O.attention_unquantized(q, lat, wl.scale)
            nmse, cos = O.int8_accuracy(r["out"], o_ref)
            rep.append((name, t, nmse, cos))
    for name, t, nmse, cos in rep:
        print(f"int8 MLA vs bf16 latents: {name} query {t}: NMSE {nmse:.3e}, cosine {cos:.7f}")
    # normal latents sit near the figures the pages report (NMSE ~5e-5, cosine
    # ~0.99997); Student-t(3) rows lose more to their per-row scale
    normal = [x for x in rep if x[0] == "decode_32k"]
    heavy = [x for x in rep if x[0] == "mini_heavy"]
    assert max(x[2] for x in normal) < 2e-4 and min(x[3] for x in normal) > 0.9999
    assert max(x[2] for x in heavy) < 5e-2 and min(x[3] for x in heavy) > 0.98
