"""Stage-by-stage parity of the HIP kernels against the oracle (GPU).

Each stage is fed seeded synthetic inputs on both sides (never a GPU result
as an oracle input) and compared element by element: INT8 rows, index lists
and top-k ids bit-exactly; pools and scores within rtol 1e-2 (absolute floor
1e-2 x row RMS); attention within max-abs 2e-2 and rel-L2 1e-2 (fp32 out).
"""
import numpy as np
import pytest
import torch

import dsa_synth as syn
import oracle as O
from oracle_chain import OracleWorkload, score_close

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_store_amd as m
    m.lib()
    return m


def dev_bf16(a):
    return torch.from_numpy(syn.bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()


def seqs_of(dsa, wl):
    return dsa.Seqs(torch.tensor(wl.first_valid, dtype=torch.int32, device="cuda"),
                    torch.tensor(wl.row_base, dtype=torch.int64, device="cuda"),
                    torch.tensor(wl.tok_base, dtype=torch.int64, device="cuda"),
                    torch.tensor(wl.pool_base, dtype=torch.int64, device="cuda"))


# ---------------------------------------------------------------- store_int8

@pytest.mark.parametrize("name", ["tiny", "mini_decode", "mini_heavy"])
def test_store_int8_bit_exact(dsa, name):
    wl = syn.get(name)
    d = wl.dims
    dims = dsa.Dims.of(d)
    say(f"store_int8 {name}")
    cache = torch.full((wl.total_rows, d.row_bytes), 0x5A, dtype=torch.int8, device="cuda")
    ref = np.full((wl.total_rows, d.row_bytes), 0x5A, dtype=np.uint8)
    for b in range(wl.B):
        n = int(wl.seq_len[b])
        lat = syn.gen_latent(wl, b, 0, n)
        slots = np.arange(n, dtype=np.int64) + wl.row_base[b]
        slots[::7] = -1                                   # padding slots are skipped
        lt = torch.from_numpy(lat).cuda() if wl.fp32_mla else dev_bf16(lat)
        dsa.store_int8(dims, lt, torch.from_numpy(slots).cuda(), cache)
        O.store_int8(lat, slots, ref)
    torch.cuda.synchronize()
    got = cache.cpu().numpy().view(np.uint8)
    assert np.array_equal(got, ref)


def test_store_int8_special_rows(dsa):
    d = syn.production_dims(16)
    dims = dsa.Dims.of(d)
    x = np.zeros((6, 512), dtype=np.float32)
    x[0, :14] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -127.0, 3.4375, 3.5625, 0.25, -126.5, 125.5]
    x[1] = 2.5                                              # constant row
    x[2] = -0.75
    # row 3: zeros (amax floor)
    x[4] = syn.bf16_round(np.linspace(-1e-5, 1e-5, 512).astype(np.float32))   # below the floor
    x[5] = syn.bf16_round((np.arange(512) % 17 - 8).astype(np.float32) * 1e3)
    assert np.array_equal(syn.bf16_round(x), x)
    slots = np.array([5, 0, 3, 1, 2, 4], dtype=np.int64)
    for dt in ("bf16", "f32"):
        say(f"store_int8 special rows {dt}")
        cache = torch.full((6, 528), 0x33, dtype=torch.int8, device="cuda")
        lt = dev_bf16(x) if dt == "bf16" else torch.from_numpy(x).cuda()
        dsa.store_int8(dims, lt, torch.from_numpy(slots).cuda(), cache)
        ref = np.zeros((6, 528), dtype=np.uint8)
        O.store_int8(x, slots, ref)
        assert np.array_equal(cache.cpu().numpy().view(np.uint8), ref)


def test_store_int8_strided_latent(dsa):
    """Rows with a leading dimension larger than D (a view into a wider buffer)."""
    d = syn.production_dims(16)
    dims = dsa.Dims.of(d)
    g = np.random.default_rng(5)
    wide = syn.bf16_round(g.standard_normal((100, 640)).astype(np.float32))
    say("store_int8 strided")
    full = dev_bf16(wide)
    cache = torch.zeros((100, 528), dtype=torch.int8, device="cuda")
    dsa.store_int8(dims, full[:, :512], torch.arange(100, dtype=torch.int64, device="cuda"), cache)
    ref = np.zeros((100, 528), dtype=np.uint8)
    O.store_int8(wide[:, :512], np.arange(100), ref)
    assert np.array_equal(cache.cpu().numpy().view(np.uint8), ref)


# ---------------------------------------------------------------- index_pools

@pytest.mark.parametrize("name", ["tiny", "tiny_seven", "tiny_padded_six", "tiny_batch", "mini_decode",
                                  "mini_prefill"])
def test_index_pools_parity(dsa, name):
    wl = syn.get(name)
    d = wl.dims
    dims = dsa.Dims.of(d)
    say(f"index_pools {name}")
    k = torch.zeros((wl.total_tokens, d.idx_dim), dtype=torch.bfloat16, device="cuda")
    gate = torch.zeros_like(k)
    for b in range(wl.B):
        kk, gg = syn.gen_kgate(wl, b, 0, int(wl.seq_len[b]))
        tb = int(wl.tok_base[b])
        k[tb:tb + kk.shape[0]] = dev_bf16(kk)
        gate[tb:tb + gg.shape[0]] = dev_bf16(gg)
    lw, lb = syn.gen_ln(wl)
    npools = max(wl.total_pools, 1) + 3
    pools = torch.full((npools, d.idx_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    ends = [wl.n_pools(b) for b in range(wl.B)]
    dsa.index_pools(dims, k, gate, torch.from_numpy(lw).cuda(), torch.from_numpy(lb).cuda(), seqs_of(dsa, wl),
                    torch.zeros(wl.B, dtype=torch.int32, device="cuda"),
                    torch.tensor(ends, dtype=torch.int32, device="cuda"), max(ends), pools)
    got = pools.float().cpu().numpy()
    ow = OracleWorkload(wl)
    written = np.zeros(npools, dtype=bool)
    for b in range(wl.B):
        ref = ow.pools(b)
        pb = int(wl.pool_base[b])
        assert ref.shape[0] == ends[b]
        for p in range(ends[b]):
            ok, worst = score_close(got[pb + p], ref[p], d.idx_dim)
            assert ok, (b, p, worst)
        written[pb:pb + ends[b]] = True
    assert np.all(got[~written] == 7.0)                     # nothing outside the listed pools


def test_index_pools_partial_range_and_f32_state(dsa):
    """A range in the middle of a sequence, k/gate given in fp32."""
    wl = syn.mini_decode()
    d = wl.dims
    dims = dsa.Dims.of(d)
    b = 1
    n = int(wl.seq_len[b])
    kk, gg = syn.gen_kgate(wl, b, 0, n)
    say("index_pools partial f32")
    k = torch.zeros((wl.total_tokens, d.idx_dim), dtype=torch.float32, device="cuda")
    gate = torch.zeros_like(k)
    tb = int(wl.tok_base[b])
    k[tb:tb + n] = torch.from_numpy(kk).cuda()
    gate[tb:tb + n] = torch.from_numpy(gg).cuda()
    lw, lb = syn.gen_ln(wl)
    pools = torch.full((wl.total_pools, d.idx_dim), 3.0, dtype=torch.bfloat16, device="cuda")
    begin = np.zeros(wl.B, dtype=np.int32)
    end = np.zeros(wl.B, dtype=np.int32)
    begin[b], end[b] = 100, 357
    dsa.index_pools(dims, k, gate, torch.from_numpy(lw).cuda(), torch.from_numpy(lb).cuda(), seqs_of(dsa, wl),
                    torch.from_numpy(begin).cuda(), torch.from_numpy(end).cuda(), 257, pools)
    got = pools.float().cpu().numpy()
    ref = OracleWorkload(wl).pools(b)
    pb = int(wl.pool_base[b])
    for p in range(100, 357):
        assert score_close(got[pb + p], ref[p], d.idx_dim)[0], p
    assert np.all(got[pb:pb + 100] == 3.0) and np.all(got[pb + 357:] == 3.0)


# ---------------------------------------------------------------- append_tokens

@pytest.mark.parametrize("name,dt,rows,pools_on", [("mini_decode", torch.bfloat16, True, True),
                                                   ("mini_prefill", torch.bfloat16, True, True),
                                                   ("mini_decode", torch.float32, True, True),
                                                   ("tiny_batch", torch.bfloat16, False, True),
                                                   ("tiny_batch", torch.bfloat16, True, False)])
def test_append_tokens_matches_separate_calls(dsa, name, dt, rows, pools_on):
    """One launch of rows + pools gives the bytes of store_int8 then index_pools."""
    wl = syn.get(name)
    d = wl.dims
    dims = dsa.Dims.of(d)
    say(f"append_tokens {name} {dt} rows={rows} pools={pools_on}")
    k = torch.zeros((wl.total_tokens, d.idx_dim), dtype=dt, device="cuda")
    gate = torch.zeros_like(k)
    for b in range(wl.B):
        kk, gg = syn.gen_kgate(wl, b, 0, int(wl.seq_len[b]))
        tb = int(wl.tok_base[b])
        if dt == torch.float32:
            k[tb:tb + kk.shape[0]] = torch.from_numpy(kk).cuda()
            gate[tb:tb + gg.shape[0]] = torch.from_numpy(gg).cuda()
        else:
            k[tb:tb + kk.shape[0]] = dev_bf16(kk)
            gate[tb:tb + gg.shape[0]] = dev_bf16(gg)
    lw, lb = syn.gen_ln(wl)
    lw, lb = torch.from_numpy(lw).cuda(), torch.from_numpy(lb).cuda()
    ends = [wl.n_pools(b) for b in range(wl.B)] if pools_on else [0] * wl.B
    begin = torch.tensor([max(e - 5, 0) for e in ends], dtype=torch.int32, device="cuda")
    end = torch.tensor(ends, dtype=torch.int32, device="cuda")
    max_pools = 5 if pools_on else 0
    n = 37 if rows else 0
    lat = syn.gen_latent(wl, 0, 0, max(n, 1))[:n]
    lt = torch.from_numpy(lat).cuda() if dt == torch.float32 else dev_bf16(lat)
    lt = lt.reshape(n, d.latent_dim)
    nrows = 64
    slots = torch.from_numpy(np.random.default_rng(3).permutation(nrows)[:n].astype(np.int64)).cuda()
    npools = max(wl.total_pools, 1) + 3
    outs = []
    for fused in (False, True):
        cache = torch.full((nrows, d.row_bytes), 0x5B, dtype=torch.int8, device="cuda")
        pools = torch.full((npools, d.idx_dim), 7.0, dtype=torch.bfloat16, device="cuda")
        if fused:
            dsa.append_tokens(dims, lt, slots, cache, k, gate, lw, lb, seqs_of(dsa, wl), begin, end, max_pools, pools)
        else:
            if n:
                dsa.store_int8(dims, lt, slots, cache)
            if max_pools:
                dsa.index_pools(dims, k, gate, lw, lb, seqs_of(dsa, wl), begin, end, max_pools, pools)
        torch.cuda.synchronize()
        outs.append((cache.cpu(), pools.view(torch.int16).cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    if rows:
        assert not torch.all(outs[1][0] == 0x5B)
    if pools_on:
        assert not torch.all(outs[1][1] == outs[1][1].flatten()[0])


# ---------------------------------------------------------------- index_scores

@pytest.mark.parametrize("name", ["tiny", "tiny_batch", "mini_decode", "mini_prefill"])
def test_index_scores_parity(dsa, name):
    """Scores from pools the oracle also uses (the oracle's fp64 pools rounded to bf16 on the host)."""
    wl = syn.get(name)
    d = wl.dims
    dims = dsa.Dims.of(d)
    ow = OracleWorkload(wl)
    npools = max(wl.total_pools, 1)
    host_pools = np.zeros((npools, d.idx_dim), dtype=np.float32)
    for b in range(wl.B):
        pb = int(wl.pool_base[b])
        pp = ow.pools(b)
        host_pools[pb:pb + pp.shape[0]] = syn.bf16_round(pp.astype(np.float32))
    stride = max(256, -(-max(wl.max_n_vis, 1) // 256) * 256) + 64
    say(f"index_scores {name} T={wl.T} stride={stride}")
    scores = torch.full((wl.T, stride), 123.0, dtype=torch.float32, device="cuda")
    qi = syn.gen_qidx(wl, 0, wl.T)
    w = syn.gen_w(wl, 0, wl.T)
    dsa.index_scores(dims, dev_bf16(qi), torch.from_numpy(w).cuda(), dev_bf16(host_pools), seqs_of(dsa, wl),
                     torch.from_numpy(wl.q_seq).cuda(), torch.from_numpy(wl.q_pos).cuda(), scores)
    got = scores.cpu().numpy()
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        n_vis = wl.n_vis(t)
        pb = int(wl.pool_base[b])
        ref = O.index_scores(qi[t], w[t], host_pools[pb:pb + n_vis].astype(np.float64), n_vis, stride)
        ok, worst = score_close(got[t], ref, n_vis, rtol=1e-4, floor=1e-4)
        assert ok, (t, worst)
        assert np.all(np.isneginf(got[t, n_vis:])), t


# ---------------------------------------------------------------- topk_select

def _topk_case(dsa, T, stride, n_vis, kind, seed, select_k=512):
    d = syn.production_dims(16)
    dims = dsa.Dims.of(d)
    sc = syn.gen_score_rows(seed, T, stride, n_vis, kind)
    fv = np.zeros(T, dtype=np.int32)
    rb = (np.arange(T, dtype=np.int64) * 1000003)
    seqs = dsa.Seqs(torch.from_numpy(fv).cuda(), torch.from_numpy(rb).cuda(),
                    torch.zeros(T, dtype=torch.int64, device="cuda"), torch.zeros(T, dtype=torch.int64, device="cuda"))
    q_seq = torch.arange(T, dtype=torch.int32, device="cuda")
    qpos_h = (np.asarray(n_vis) * 4 + (np.arange(T) % 4) - 1).astype(np.int32)   # n_vis pools + tail 0..3
    q_pos = torch.from_numpy(qpos_h).cuda()
    ws = dsa.topk_workspace(dims, T, stride)
    scd = torch.from_numpy(sc).cuda()
    out = torch.full((T, select_k), 77777, dtype=torch.int32, device="cuda")
    dsa.topk_select(dims, scd, seqs, q_seq, q_pos, out, ws)
    got1 = out.cpu().numpy()
    out.fill_(-5)
    idx = torch.full((T, d.out_width), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    dsa.topk_select_expand(dims, scd, seqs, q_seq, q_pos, idx, out, ws)      # workspace reused without clearing
    got2 = out.cpu().numpy()
    gidx = idx.cpu().numpy()
    assert np.array_equal(got1, got2)
    for t in range(T):
        assert O.visible_pool_count(int(qpos_h[t]), 0, 4) == int(n_vis[t])
        ref = O.topk_pools(sc[t].astype(np.float64), int(n_vis[t]), select_k)
        assert np.array_equal(got1[t], ref), (kind, t, int(n_vis[t]))
        ref_idx = O.expand_selection(ref, 0, int(qpos_h[t]), int(rb[t]), d.kpool, d.out_width)
        assert np.array_equal(gidx[t], ref_idx), (kind, t)
    return ws is not None


@pytest.mark.parametrize("kind", ["ties", "normal", "equal", "signed_zero"])
def test_topk_rows_up_to_65536(dsa, kind):
    n_vis = np.array([0, 1, 300, 511, 512, 513, 600, 2000, 8192, 20000, 33792, 65535, 65536, 63639],
                     dtype=np.int64)
    say(f"topk row {kind}")
    _topk_case(dsa, len(n_vis), 65536, n_vis, kind, seed=21)


@pytest.mark.parametrize("kind", ["ties", "normal", "equal", "signed_zero"])
def test_topk_rows_past_65536(dsa, kind):
    n_vis = np.array([0, 512, 513, 4097, 65536, 40000, 70000, 69999, 12345], dtype=np.int64)
    say(f"topk long {kind}")
    _topk_case(dsa, len(n_vis), 70000, n_vis, kind, seed=22)


@pytest.mark.parametrize("kind", ["ties", "normal", "equal", "signed_zero"])
def test_topk_rows_single_pass(dsa, kind):
    """Rows of up to 40,960 pools are selected in one pass over their scores
    (no workspace); 40,964 takes the tile path."""
    n_vis = np.array([0, 1, 511, 512, 513, 2000, 20000, 40959, 40960, 33792], dtype=np.int64)
    say(f"topk single pass {kind}")
    assert dsa.topk_workspace_bytes(dsa.Dims.of(syn.production_dims(16)), len(n_vis), 40960) == 0
    _topk_case(dsa, len(n_vis), 40960, n_vis, kind, seed=25)
    _topk_case(dsa, 3, 40964, np.array([40964, 40961, 600], dtype=np.int64), kind, seed=26)


def test_topk_rows_of_262144(dsa):
    n_vis = np.array([262144, 262143, 384, 1], dtype=np.int64)
    say("topk long 262144")
    _topk_case(dsa, 4, 262144, n_vis, "ties", seed=23)


def test_topk_odd_stride_scalar_loads(dsa):
    n_vis = np.array([1001, 999, 3], dtype=np.int64)
    say("topk odd stride")
    _topk_case(dsa, 3, 1001, n_vis, "normal", seed=24)


# ---------------------------------------------------------------- expand_selection

@pytest.mark.parametrize("name", ["tiny", "tiny_batch", "mini_decode", "mini_prefill"])
def test_expand_parity(dsa, name):
    wl = syn.get(name)
    d = wl.dims
    dims = dsa.Dims.of(d)
    g = np.random.default_rng(31)
    ids = np.full((wl.T, d.select_k), -1, dtype=np.int32)
    for t in range(wl.T):
        n_vis = wl.n_vis(t)
        k = min(d.select_k, n_vis)
        ids[t, :k] = np.sort(g.choice(n_vis, size=k, replace=False)) if k else []
    say(f"expand {name}")
    out = torch.full((wl.T, d.out_width), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    dsa.expand_selection(dims, torch.from_numpy(ids).cuda(), seqs_of(dsa, wl), torch.from_numpy(wl.q_seq).cuda(),
                         torch.from_numpy(wl.q_pos).cuda(), out)
    got = out.cpu().numpy()
    assert not np.any(got == 0x7F7F7F7F)
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        ref = O.expand_selection(ids[t], int(wl.first_valid[b]), int(wl.q_pos[t]), int(wl.row_base[b]),
                                 d.kpool, d.out_width)
        assert np.array_equal(got[t], ref), t


# ---------------------------------------------------------------- sparse_mla

def _mla_case(dsa, wl, T, valid, num_splits, out_dtype=torch.float32, seed=41):
    d = wl.dims
    dims = dsa.Dims.of(d)
    rows = wl.total_rows
    lat = np.concatenate([syn.gen_latent(wl, b, 0, int(wl.seq_len[b])) for b in range(wl.B)])
    # All sequences stored back to back at their row bases.
    slots = np.concatenate([np.arange(int(wl.seq_len[b])) + int(wl.row_base[b]) for b in range(wl.B)])
    ref_cache = np.zeros((rows, d.row_bytes), dtype=np.uint8)
    O.store_int8(lat, slots, ref_cache)
    cache = torch.from_numpy(ref_cache.view(np.int8)).cuda()      # oracle bytes, bit-identical to store_int8's
    lists = syn.gen_index_lists(seed, T, d.out_width, syn.valid_rows(wl), valid)
    q = np.concatenate([syn.gen_q(wl, 0, wl.T)] * (-(-T // wl.T)))[:T]
    qd = torch.from_numpy(q).cuda() if wl.fp32_mla else dev_bf16(q)
    out = torch.full((T, d.mla_heads, d.latent_dim), 99.0, dtype=out_dtype, device="cuda")
    lse = torch.full((T, d.mla_heads), 99.0, dtype=torch.float32, device="cuda")
    n = dsa.sparse_mla_workspace_bytes(dims, T, num_splits)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    say(f"sparse_mla {wl.name} T={T} splits={num_splits} out={out_dtype}")
    dsa.sparse_mla(dims, qd, cache, torch.from_numpy(lists).cuda(), wl.scale, out, lse, num_splits, ws)
    o1 = out.float().cpu().numpy()
    l1 = lse.cpu().numpy()
    dsa.sparse_mla(dims, qd, cache, torch.from_numpy(lists).cuda(), wl.scale, out, lse, num_splits, ws)
    assert np.array_equal(out.float().cpu().numpy(), o1)         # bitwise run-to-run determinism
    refs = [O.sparse_mla(q[t], ref_cache, lists[t], wl.scale, d.latent_dim) for t in range(T)]
    ro = np.stack([r[0] for r in refs])
    rl = np.stack([r[1] for r in refs])
    extra = 0.0
    if out_dtype == torch.bfloat16:
        extra = np.abs(ro) * 2.0 ** -8                              # half a bf16 ulp of |o|
    err = np.abs(o1 - ro)
    assert np.all(err <= 2e-2 + extra), float(err.max())
    if np.any(valid > 0):
        rel = np.linalg.norm(o1 - ro) / np.linalg.norm(ro)
        assert rel <= 1e-2, rel
    empty = valid == 0
    assert np.all(o1[empty] == 0) and np.all(np.isneginf(l1[empty]))
    fin = ~empty
    assert np.allclose(l1[fin], rl[fin], atol=2e-3, rtol=1e-4)
    return o1


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_sparse_mla_decode_h16(dsa, splits):
    wl = syn.mini_decode()
    valid = np.array([2051, 2048, 0, 1, 7, 64, 65, 1000, 2176, 2049, 130, 511], dtype=np.int64)
    _mla_case(dsa, wl, len(valid), valid, splits)


def test_sparse_mla_split_count_invariance(dsa):
    wl = syn.mini_decode()
    valid = np.array([2051, 1500, 3, 2176], dtype=np.int64)
    a = _mla_case(dsa, wl, 4, valid, 1)
    b = _mla_case(dsa, wl, 4, valid, 7)
    assert np.allclose(a, b, atol=1e-5, rtol=1e-4)


def test_sparse_mla_h64_small_batch(dsa):
    wl = syn.mini_heavy()
    valid = np.array([2049, 1537, 6, 0], dtype=np.int64)
    _mla_case(dsa, wl, 4, valid, 0)


@pytest.mark.parametrize("splits", [1, 3])
def test_sparse_mla_h64_prefill_tiles(dsa, splits):
    """The many-query kernel (64 heads a workgroup, 8 waves), whole lists per
    workgroup or split with partials and the merge."""
    wl = syn.mini_heavy()
    g = np.random.default_rng(3)
    valid = g.integers(0, 2177, size=160)
    valid[:3] = [0, 2176, 2051]
    _mla_case(dsa, wl, 160, valid, splits)


@pytest.mark.parametrize("splits", [1, 2])
def test_sparse_mla_h32_prefill_tiles(dsa, splits):
    """32 heads over many queries: the many-query kernel with two 16-head
    tiles a workgroup (k_mla_mfma<2, 4>)."""
    import dataclasses
    wl = syn.mini_heavy()
    wl = dataclasses.replace(wl, dims=syn.production_dims(32), name="mini_heavy_h32")
    g = np.random.default_rng(5)
    valid = g.integers(0, 2177, size=300)
    valid[:3] = [0, 2176, 1]
    _mla_case(dsa, wl, 300, valid, splits)


@pytest.mark.parametrize("heads,T,splits", [(64, 160, 1), (64, 160, 3), (16, 6, 0)])
def test_sparse_mla_ragged_width(dsa, heads, T, splits):
    """Lists 2,100 wide: a 52-row last chunk for both the many-query kernel
    (64-row chunks, k_mla_mfma at 64 heads and 160 queries) and the decode
    kernel (128-row chunks, 16 heads), empty slots past the width included."""
    import dataclasses
    wl = syn.mini_heavy() if heads == 64 else syn.mini_decode()
    wl = dataclasses.replace(wl, dims=dataclasses.replace(wl.dims, out_width=2100), name=wl.name + "_w2100")
    g = np.random.default_rng(11)
    valid = g.integers(0, 2101, size=T)
    valid[:3] = [2100, 0, 2099]
    _mla_case(dsa, wl, T, valid, splits)


def test_sparse_mla_bf16_output(dsa):
    wl = syn.mini_decode()
    valid = np.array([2051, 100, 0, 2176], dtype=np.int64)
    _mla_case(dsa, wl, 4, valid, 0, out_dtype=torch.bfloat16)


def test_sparse_mla_tiny_fp32(dsa):
    wl = syn.tiny()
    valid = np.array([0, 1, 5, 19, 24, 16] * 3, dtype=np.int64)
    _mla_case(dsa, wl, len(valid), valid, 0)


# ---------------------------------------------------------------- scoring with group lists

def _scores_select_case(name, zero_q=False):
    import dsa_harness
    wl = syn.get(name)
    dw = dsa_harness.DeviceWorkload(wl)
    if zero_q:
        dw.q_idx.zero_()                     # all-equal scores: every group certificate fails
    dw.step_calls()                          # index_scores + topk_select_expand, one call each
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dw.scores, dw.pool_ids, dw.indices)]
    for x in (dw.pool_ids, dw.indices):
        x.fill_(0x5A5A5A5A)
    dw.scores.fill_(float("nan"))
    dw.step_scores_select()
    torch.cuda.synchronize()
    for nm, a, b in zip(("scores", "pool_ids", "indices"), ref, (dw.scores, dw.pool_ids, dw.indices)):
        assert torch.equal(a, b), nm


@pytest.mark.parametrize("name", ["mini_decode", "mini_heavy", "decode_32k", "mini_long"])
def test_index_scores_select_matches_separate_calls(dsa, name):
    """The group-list selection (64- or 256-pool groups) against the tile
    selection over the full score rows: the same bits."""
    say(f"index_scores_select {name}")
    _scores_select_case(name)


@pytest.mark.parametrize("name", ["decode_32k", "mini_long"])
def test_index_scores_select_forced_fallback(dsa, name):
    say(f"index_scores_select with all-equal scores {name}")
    _scores_select_case(name, zero_q=True)
