"""Paged caches (blocks of 256 positions through a block table, a seeded
permutation of physical blocks with spare blocks) against the flat layout:
the paged decode step (dsa_harness.PagedWorkload.step: store_int8 at the
physical slots, index_pools_paged, index_scores_groups_paged,
topk_select_groups_paged, sparse_mla) gives the flat step's pools, scores,
pool ids and attention bit for bit, and an index list that is the flat one
mapped through the block table; the flat step is checked against the oracle
by the chain tests.  Left padding that is not a multiple of 4 makes some
pools straddle two blocks."""
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


@pytest.mark.parametrize("name", ["mini_decode", "mini_decode_64", "mini_heavy", "mini_mtp",
                                  pytest.param("decode_262k_b8", marks=pytest.mark.slow)])
def test_paged_step_matches_flat(harness, name):
    wl = syn.get(name)
    say(f"paged {name}")
    pw = harness.PagedWorkload(wl)
    fw = harness.DeviceWorkload(wl)
    pw.step()
    fw.step_append()
    fw.step_scores_groups()
    fw.step_select_groups()
    fw.step_attention()
    torch.cuda.synchronize()
    # pools: every pool of every sequence at its paged row
    fp, pp = fw.pools[0].view(torch.int16).cpu().numpy(), pw.pools.view(torch.int16).cpu().numpy()
    for b in range(wl.B):
        n = wl.n_pools(b)
        p = np.arange(n)
        prow = pw.table_np[b, p >> 6].astype(np.int64) * 64 + (p & 63)
        assert np.array_equal(pp[prow], fp[int(wl.pool_base[b]) + p]), ("pools", b)
    for what in ("scores", "pool_ids", "out", "lse"):
        assert torch.equal(getattr(fw, what), getattr(pw, what)), what
    fi, pi = fw.indices.cpu().numpy().astype(np.int64), pw.indices.cpu().numpy().astype(np.int64)
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        v = fi[t]
        want = np.where(v >= 0, pw.rows(b, np.maximum(v - int(wl.row_base[b]), 0)), -1)
        assert np.array_equal(pi[t], want), ("indices", t)
        # the rows the paged list names hold the flat rows' bytes
        valid = v[v >= 0]
        if valid.size:
            a = fw.caches[0][torch.from_numpy(valid).cuda()]
            c = pw.cache[torch.from_numpy(pi[t][pi[t] >= 0]).cuda()]
            assert torch.equal(a, c), ("rows", t)
