"""Host-only checks of the C ABI (no GPU needed, nothing is launched).

The shared library must load, export every function include/dsa.h declares,
and reject invalid host-visible arguments with the documented status codes
before touching the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, E_NULL, E_DIMS, E_DTYPE, E_ALIGN, E_WIDTH, E_WS, E_UNSUP, E_HIP, E_SIZE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_store_amd as m
    if not os.path.exists(m.LIB_PATH):
        from sparse_attention_store_amd import build
        build.build(verbose=False)
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path_calls():
    names = declared_functions()
    for want in ["dsa_store_int8", "dsa_index_pools", "dsa_index_scores", "dsa_topk_select",
                 "dsa_topk_select_expand", "dsa_expand_selection", "dsa_sparse_mla",
                 "dsa_topk_workspace_bytes", "dsa_sparse_mla_workspace_bytes", "dsa_status_string",
                 "dsa_abi_version"]:
        assert want in names


def test_library_exports_every_declared_symbol(dsa):
    L = dsa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dsa_[a-z0-9_]+)\b", out))
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in exported, name


def test_version_and_status_strings(dsa):
    assert dsa.abi_version() == 1
    for code in (OK, E_NULL, E_DIMS, E_DTYPE, E_ALIGN, E_WIDTH, E_WS, E_UNSUP, E_HIP, E_SIZE):
        assert dsa.status_string(code) and dsa.status_string(code) != "unknown status"
    assert dsa.status_string(-123) == "unknown status"


def prod(dsa, **kw):
    v = dict(idx_heads=32, idx_dim=128, kpool=4, index_topk=2048, out_width=2176, mla_heads=16,
             latent_dim=512, row_bytes=528, ln_eps=1e-5)
    v.update(kw)
    return dsa.Dims(*[v[k] for k in ["idx_heads", "idx_dim", "kpool", "index_topk", "out_width", "mla_heads",
                                     "latent_dim", "row_bytes", "ln_eps"]])


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every case below fails validation first
MISALIGNED = ctypes.c_void_p(0x10008)


def seqs(dsa, ptr=FAKE):
    return dsa._Seqs(ptr, ptr, ptr, ptr)


def test_dims_validation(dsa):
    L = dsa.lib()
    store = lambda d: L.dsa_store_int8(ctypes.byref(d) if d is not None else None, FAKE, 1, 1, 512, FAKE, FAKE, 1, None)
    assert L.dsa_store_int8(None, FAKE, 1, 1, 512, FAKE, FAKE, 1, None) == E_NULL
    assert store(prod(dsa, idx_heads=0)) == E_DIMS
    assert store(prod(dsa, index_topk=2047)) == E_DIMS                 # not a multiple of kpool
    assert store(prod(dsa, row_bytes=520)) == E_DIMS                   # must be round_up(D + 4, 16)
    assert store(prod(dsa, out_width=2050)) == E_WIDTH                 # < index_topk + kpool - 1
    assert store(prod(dsa, ln_eps=-1.0)) == E_DIMS


def test_append_tokens_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    S = seqs(dsa)
    call = lambda dt=1, lat=FAKE, n=4, ld=512, sl=FAKE, c=FAKE, k=FAKE, mp=2, sq=ctypes.byref(S), dims=bd: \
        L.dsa_append_tokens(dims, dt, lat, n, ld, sl, c, 64, k, FAKE, FAKE, FAKE, sq, 2, FAKE, FAKE, mp, FAKE, None)
    assert call(dims=None) == E_NULL
    assert call(dims=ctypes.byref(prod(dsa, idx_heads=0))) == E_DIMS
    assert call(dt=7) == E_DTYPE
    assert call(dims=ctypes.byref(prod(dsa, latent_dim=96, row_bytes=112))) == E_UNSUP
    assert call(dims=ctypes.byref(prod(dsa, idx_dim=64))) == E_UNSUP
    assert call(n=-1) == E_SIZE
    assert call(mp=-1) == E_SIZE
    assert call(lat=None) == E_NULL
    assert call(ld=500) == E_SIZE
    assert call(lat=MISALIGNED) == E_ALIGN
    assert call(k=None) == E_NULL
    assert call(k=ctypes.c_void_p(0x10002)) == E_ALIGN          # k and gate need 4-byte alignment
    assert call(sq=None) == E_NULL
    # nothing to do: no launch, no pointer needed
    assert call(n=0, mp=0, lat=None, sl=None, c=None, k=None, sq=None) == OK


def test_append_scores_groups_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    S = seqs(dsa)
    ws_need = L.dsa_index_scores_select_workspace_bytes(bd, 8, 65536)
    assert ws_need > 0

    def call(dims=bd, dt=1, lat=FAKE, n=8, mp=1, k=FAKE, q_idx=FAKE, sq=ctypes.byref(S), T=8, stride=65536,
             ws=FAKE, ws_bytes=ws_need):
        return L.dsa_append_scores_groups(dims, dt, lat, n, 512, FAKE, FAKE, 64, k, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          mp, FAKE, q_idx, FAKE, sq, 8, FAKE, FAKE, T, stride, FAKE, ws, ws_bytes,
                                          None)
    assert call(dims=None) == E_NULL
    assert call(dt=7) == E_DTYPE
    assert call(dims=ctypes.byref(prod(dsa, idx_dim=64))) == E_UNSUP
    assert call(n=-1) == E_SIZE
    assert call(lat=None) == E_NULL
    assert call(lat=MISALIGNED) == E_ALIGN
    assert call(ws_bytes=ws_need - 1) == E_WS
    assert call(ws=None) == E_WS
    assert call(T=65) == E_UNSUP                                # no group lists for more than 64 queries
    assert call(sq=None) == E_NULL
    assert call(k=None) == E_NULL
    assert call(k=ctypes.c_void_p(0x10002)) == E_ALIGN
    assert call(q_idx=None) == E_NULL
    assert call(q_idx=MISALIGNED) == E_ALIGN
    # nothing to do: no launch
    assert call(n=0, mp=0, T=0, lat=None, k=None, q_idx=None, ws=None, ws_bytes=0) == OK


def test_store_int8_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    assert L.dsa_store_int8(bd, FAKE, 7, 1, 512, FAKE, FAKE, 1, None) == E_DTYPE
    assert L.dsa_store_int8(bd, FAKE, 1, -1, 512, FAKE, FAKE, 1, None) == E_SIZE
    assert L.dsa_store_int8(bd, FAKE, 1, 0, 512, None, None, 0, None) == OK       # nothing to do
    assert L.dsa_store_int8(bd, None, 1, 4, 512, FAKE, FAKE, 4, None) == E_NULL
    assert L.dsa_store_int8(bd, FAKE, 1, 4, 500, FAKE, FAKE, 4, None) == E_SIZE  # ld < D
    assert L.dsa_store_int8(bd, MISALIGNED, 1, 4, 512, FAKE, FAKE, 4, None) == E_ALIGN
    assert L.dsa_store_int8(bd, FAKE, 1, 4, 516, FAKE, FAKE, 4, None) == E_ALIGN  # row pitch not 16 B
    d2 = prod(dsa, latent_dim=320, row_bytes=336)
    assert L.dsa_store_int8(ctypes.byref(d2), FAKE, 1, 4, 320, FAKE, FAKE, 4, None) == E_UNSUP


def test_pools_scores_expand_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    s = seqs(dsa)
    assert L.dsa_index_pools(bd, FAKE, FAKE, 9, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 1, FAKE, None) == E_DTYPE
    d3 = prod(dsa, idx_dim=64)
    assert L.dsa_index_pools(ctypes.byref(d3), FAKE, FAKE, 1, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 1, FAKE,
                             None) == E_UNSUP
    assert L.dsa_index_pools(bd, FAKE, FAKE, 1, FAKE, FAKE, None, 1, FAKE, FAKE, 1, FAKE, None) == E_NULL
    assert L.dsa_index_pools(bd, FAKE, FAKE, 1, FAKE, FAKE, ctypes.byref(s), 0, FAKE, FAKE, 1, FAKE, None) == E_SIZE
    assert L.dsa_index_pools(bd, None, FAKE, 1, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 1, FAKE, None) == E_NULL
    assert L.dsa_index_pools(bd, FAKE, FAKE, 1, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 0, FAKE, None) == OK
    assert L.dsa_index_scores(bd, FAKE, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, -1, 256, FAKE, None) == E_SIZE
    assert L.dsa_index_scores(bd, None, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 4, 256, FAKE, None) == E_NULL
    assert L.dsa_index_scores(bd, MISALIGNED, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 4, 256, FAKE,
                              None) == E_ALIGN
    assert L.dsa_index_scores(bd, FAKE, FAKE, FAKE, ctypes.byref(s), 1, FAKE, FAKE, 0, 256, FAKE, None) == OK
    assert L.dsa_expand_selection(bd, None, ctypes.byref(s), 1, FAKE, FAKE, 4, FAKE, None) == E_NULL
    sn = dsa._Seqs(FAKE, None, FAKE, FAKE)
    assert L.dsa_expand_selection(bd, FAKE, ctypes.byref(sn), 1, FAKE, FAKE, 4, FAKE, None) == E_NULL


def test_topk_argument_checks_and_workspace(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    s = seqs(dsa)
    need = L.dsa_topk_workspace_bytes(bd, 8, 65536)
    assert need > 0 and L.dsa_topk_workspace_bytes(bd, 8, 65536 * 2) > need
    assert L.dsa_topk_select(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 8, FAKE, FAKE, need - 1,
                             None) == E_WS
    assert L.dsa_topk_select(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 8, FAKE, None, need, None) == E_WS
    assert L.dsa_topk_select(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 8, FAKE, MISALIGNED, need,
                             None) == E_ALIGN
    assert L.dsa_topk_select(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 8, None, FAKE, need, None) == E_NULL
    assert L.dsa_topk_select(bd, FAKE, 300000, ctypes.byref(s), 1, FAKE, FAKE, 8, FAKE, FAKE, 1 << 30,
                             None) == E_UNSUP                               # past the 262,144-pool limit
    assert L.dsa_topk_select_expand(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 8, None, None, FAKE, need,
                                    None) == E_NULL
    assert L.dsa_topk_select(bd, FAKE, 65536, ctypes.byref(s), 1, FAKE, FAKE, 0, FAKE, None, 0, None) == OK


def test_sparse_mla_argument_checks_and_workspace(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    assert L.dsa_sparse_mla_workspace_bytes(bd, 8, 1) == 0                   # one split: no partials
    need = L.dsa_sparse_mla_workspace_bytes(bd, 8, 5)
    assert need == 8 * 5 * 16 * (512 * 4 + 8)
    assert L.dsa_sparse_mla(bd, FAKE, 5, FAKE, 10, FAKE, 8, 0.04, FAKE, 0, None, 0, FAKE, 1 << 30, None) == E_DTYPE
    assert L.dsa_sparse_mla(bd, FAKE, 1, FAKE, 10, FAKE, 8, 0.04, FAKE, 3, None, 0, FAKE, 1 << 30, None) == E_DTYPE
    assert L.dsa_sparse_mla(bd, FAKE, 1, FAKE, 10, FAKE, -1, 0.04, FAKE, 0, None, 0, FAKE, 1 << 30, None) == E_SIZE
    assert L.dsa_sparse_mla(bd, None, 1, FAKE, 10, FAKE, 8, 0.04, FAKE, 0, None, 0, FAKE, 1 << 30, None) == E_NULL
    assert L.dsa_sparse_mla(bd, MISALIGNED, 1, FAKE, 10, FAKE, 8, 0.04, FAKE, 0, None, 0, FAKE, 1 << 30,
                            None) == E_ALIGN
    assert L.dsa_sparse_mla(bd, FAKE, 1, FAKE, 10, FAKE, 8, 0.04, FAKE, 0, None, 5, FAKE, need - 1,
                            None) == E_WS
    assert L.dsa_sparse_mla(bd, FAKE, 1, FAKE, 10, FAKE, 70000, 0.04, FAKE, 0, None, 1, None, 0, None) == E_SIZE
    d4 = prod(dsa, latent_dim=2048, row_bytes=2064)
    assert L.dsa_sparse_mla(ctypes.byref(d4), FAKE, 1, FAKE, 10, FAKE, 8, 0.04, FAKE, 0, None, 1, None, 0,
                            None) == E_UNSUP


def test_binding_refuses_host_tensors(dsa):
    import torch
    d = prod(dsa)
    with pytest.raises((TypeError, ValueError)):
        dsa.store_int8(d, torch.zeros(2, 512, dtype=torch.bfloat16), torch.zeros(2, dtype=torch.int64),
                       torch.zeros(2, 528, dtype=torch.int8))


def test_time_next_scoring_launch_argument_checks(dsa):
    """The timing hook takes both events or neither (no GPU call is made)."""
    L = dsa.lib()
    assert L.dsa_time_next_scoring_launch(FAKE, None) == -1
    assert L.dsa_time_next_scoring_launch(None, FAKE) == -1
    assert L.dsa_time_next_scoring_launch(None, None) == 0


def test_topk_sparse_mla_argument_checks(dsa):
    """dsa_topk_sparse_mla checks what dsa_topk_select_groups and dsa_sparse_mla
    check (host-visible arguments only; every call here fails before a launch,
    except T = 0, which has nothing to do)."""
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    S = seqs(dsa)
    ws_need = L.dsa_index_scores_select_workspace_bytes(bd, 8, 65536)
    mla_need = L.dsa_sparse_mla_workspace_bytes(bd, 8, 17)
    assert ws_need > 0 and mla_need > 0

    def call(dims=bd, stride=65536, sq=ctypes.byref(S), T=8, idx=FAKE, ws=FAKE, ws_bytes=ws_need, q=FAKE,
             q_dt=1, out=FAKE, out_dt=0, splits=17, mws=FAKE, mws_bytes=mla_need, scores=FAKE):
        return L.dsa_topk_sparse_mla(dims, scores, stride, sq, 8, FAKE, FAKE, T, FAKE, idx, ws, ws_bytes, q, q_dt,
                                     FAKE, 1 << 20, 0.044, out, out_dt, FAKE, splits, mws, mws_bytes, None)
    assert call(dims=None) == E_NULL
    assert call(sq=None) == E_NULL
    assert call(T=65) == E_UNSUP                      # group lists: at most 64 queries
    assert call(stride=0) == E_UNSUP                  # no lists without pools
    assert call(ws_bytes=ws_need - 1) == E_WS
    assert call(idx=None) == E_NULL
    assert call(scores=None) == E_NULL
    assert call(q_dt=7) == E_DTYPE
    assert call(out_dt=7) == E_DTYPE
    assert call(splits=-1) == E_SIZE
    assert call(q=None) == E_NULL
    assert call(q=MISALIGNED) == E_ALIGN
    assert call(mws=None) == E_WS
    assert call(mws_bytes=mla_need - 1) == E_WS
    assert call(T=0, idx=None, ws=None, ws_bytes=0) == OK


def test_chunked_selection_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    s = ctypes.byref(seqs(dsa))
    # workspace size: one chunk's fp32 scores (rounded to 256 B) plus the top-k scratch of one chunk
    n = L.dsa_index_select_chunked_workspace_bytes(bd, 512, 33792)
    assert n >= 512 * 33792 * 4 and n < 512 * 33792 * 4 + (64 << 20)
    assert L.dsa_index_select_chunked_workspace_bytes(bd, 0, 33792) == 0
    args = [bd, FAKE, FAKE, FAKE, s, 1, FAKE, FAKE, 4096, 33792, 512, FAKE, FAKE, FAKE, n, None]
    bad = list(args)
    bad[10] = 0                                            # chunk
    assert L.dsa_index_select_chunked(*bad) == E_SIZE
    bad = list(args)
    bad[12] = None                                         # indices
    assert L.dsa_index_select_chunked(*bad) == E_NULL
    bad = list(args)
    bad[14] = n - 1                                        # workspace too small
    assert L.dsa_index_select_chunked(*bad) == E_WS
    bad = list(args)
    bad[1] = MISALIGNED
    assert L.dsa_index_select_chunked(*bad) == E_ALIGN
    bad = list(args)
    bad[8] = 0                                             # no queries: nothing to do
    assert L.dsa_index_select_chunked(*bad) == OK


def test_decode_step_status_argument_checks(dsa):
    L = dsa.lib()
    assert L.dsa_decode_step_status(None, 64, None) == E_NULL
    assert L.dsa_decode_step_status(FAKE, 8, None) == E_WS
    for code in (-10, -11):
        assert dsa.status_string(code) != "unknown status"


def test_int8_pool_argument_checks(dsa):
    L = dsa.lib()
    d = prod(dsa)
    bd = ctypes.byref(d)
    s = ctypes.byref(seqs(dsa))
    # pool build: dtype, unsupported geometry, missing scales, misaligned codes
    assert L.dsa_index_pools_int8(bd, FAKE, FAKE, 9, FAKE, FAKE, s, 1, FAKE, FAKE, 4, FAKE, FAKE, None, None) == E_DTYPE
    d64 = prod(dsa, idx_dim=64)
    assert L.dsa_index_pools_int8(ctypes.byref(d64), FAKE, FAKE, 1, FAKE, FAKE, s, 1, FAKE, FAKE, 4, FAKE, FAKE, None,
                                  None) == E_UNSUP
    assert L.dsa_index_pools_int8(bd, FAKE, FAKE, 1, FAKE, FAKE, s, 1, FAKE, FAKE, 4, FAKE, None, None, None) == E_NULL
    assert L.dsa_index_pools_int8(bd, FAKE, FAKE, 1, FAKE, FAKE, s, 1, FAKE, FAKE, 4, MISALIGNED, FAKE, None,
                                  None) == E_ALIGN
    assert L.dsa_index_pools_int8(bd, FAKE, FAKE, 1, FAKE, FAKE, s, 1, FAKE, FAKE, 0, FAKE, FAKE, None, None) == OK
    # scoring: decode shapes only (at most 64 queries)
    assert L.dsa_index_scores_int8(bd, FAKE, FAKE, FAKE, FAKE, s, 1, FAKE, FAKE, 65, 256, FAKE, None) == E_UNSUP
    assert L.dsa_index_scores_int8(bd, FAKE, FAKE, None, FAKE, s, 1, FAKE, FAKE, 4, 256, FAKE, None) == E_NULL
    assert L.dsa_index_scores_int8(bd, FAKE, FAKE, MISALIGNED, FAKE, s, 1, FAKE, FAKE, 4, 256, FAKE, None) == E_ALIGN
    ws = L.dsa_index_scores_select_workspace_bytes(bd, 4, 256)
    assert L.dsa_index_scores_groups_int8(bd, FAKE, FAKE, FAKE, FAKE, s, 1, FAKE, FAKE, 4, 256, FAKE, FAKE, ws - 1,
                                          None) == E_WS
    # the single launch: bf16 new tokens only
    args = [bd, 1, FAKE, 4, 512, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, s, 1,
            FAKE, FAKE, 4, 256, FAKE, FAKE, ws, None]
    bad = list(args)
    bad[1] = 0
    assert L.dsa_append_scores_groups_int8(*bad) == E_UNSUP
    bad = list(args)
    bad[16] = None                                         # scales
    assert L.dsa_append_scores_groups_int8(*bad) == E_NULL
