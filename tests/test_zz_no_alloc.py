"""dsa_sparse_mla_noalloc (split partials in the library's fixed device
array) against dsa_sparse_mla (partials in a caller workspace): the same
kernels, so the same bits, on two calls in a row, the second with a smaller
input; and a call too large for the fixed array is refused."""
import ctypes

import numpy as np
import pytest
import torch

import dsa_synth as syn

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_store_amd as dsa
    L = dsa.lib()
    wl = syn.mini_decode()
    d = wl.dims
    dims = dsa.Dims.of(d)
    rows = wl.total_rows
    say("no-alloc sparse_mla: cache of mini_decode")
    cache = torch.zeros((rows, d.row_bytes), dtype=torch.int8, device="cuda")
    for b in range(wl.B):
        n = int(wl.seq_len[b])
        lat = torch.from_numpy(syn.bf16_bits(syn.gen_latent(wl, b, 0, n)).view(np.int16)).view(torch.bfloat16).cuda()
        slots = torch.arange(int(wl.row_base[b]), int(wl.row_base[b]) + n, dtype=torch.int64, device="cuda")
        dsa.store_int8(dims, lat, slots, cache)
    stream = torch.cuda.current_stream()
    # a larger call, then a smaller one: the second must not see the first's partials
    for T, splits, seed in ((40, 0, 3), (24, 17, 4), (6, 5, 5)):
        valid = np.random.default_rng(seed).integers(0, d.out_width + 1, size=T)
        valid[0] = 0                                  # an empty list
        valid[-1] = d.out_width                       # a full one
        lists = torch.from_numpy(syn.gen_index_lists(seed, T, d.out_width, syn.valid_rows(wl), valid)).cuda()
        qn = syn.gen_q(wl, 0, wl.T)
        q = np.concatenate([qn] * (-(-T // wl.T)))[:T]
        q = torch.from_numpy(syn.bf16_bits(q).view(np.int16)).view(torch.bfloat16).cuda().contiguous()
        n = dsa.sparse_mla_workspace_bytes(dims, T, splits)
        assert 0 < n <= dsa.sparse_mla_noalloc_scratch_bytes()
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        outs = []
        for noalloc in (False, True):
            out = torch.full((T, d.mla_heads, d.latent_dim), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((T, d.mla_heads), float("nan"), dtype=torch.float32, device="cuda")
            say(f"no-alloc sparse_mla T={T} splits={splits} noalloc={noalloc}")
            if noalloc:
                st = L.dsa_sparse_mla_noalloc(ctypes.byref(dims), q.data_ptr(), dsa.DSA_BF16, cache.data_ptr(), rows,
                                              lists.data_ptr(), T, float(wl.scale), out.data_ptr(), dsa.DSA_F32,
                                              lse.data_ptr(), splits, ctypes.c_void_p(stream.cuda_stream))
            else:
                st = L.dsa_sparse_mla(ctypes.byref(dims), q.data_ptr(), dsa.DSA_BF16, cache.data_ptr(), rows,
                                      lists.data_ptr(), T, float(wl.scale), out.data_ptr(), dsa.DSA_F32,
                                      lse.data_ptr(), splits, ws.data_ptr(), n, ctypes.c_void_p(stream.cuda_stream))
            assert st == 0, L.dsa_status_string(st)
            torch.cuda.synchronize()
            outs.append((out.cpu(), lse.cpu()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), (T, splits)
        assert torch.all(outs[1][0][0] == 0) and torch.all(torch.isneginf(outs[1][1][0]))


def test_noalloc_refuses_calls_beyond_its_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_store_amd as dsa
    L = dsa.lib()
    dims = dsa.Dims.of(syn.production_dims(64))
    T = 4096                                          # 4096 x splits x 64 heads of partials: far beyond 16 MiB
    assert dsa.sparse_mla_workspace_bytes(dims, T, 8) > dsa.sparse_mla_noalloc_scratch_bytes()
    fake = 1 << 20
    st = L.dsa_sparse_mla_noalloc(ctypes.byref(dims), fake, dsa.DSA_BF16, fake, 1, fake, T, 0.05, fake,
                                  dsa.DSA_F32, None, 8, None)
    assert st == -11, L.dsa_status_string(st)
