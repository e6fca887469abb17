"""The bounded-workspace selection for many queries (dsa_index_select_chunked)
against the unbounded calls (dsa_index_scores over all queries, then
dsa_topk_select_expand): the same pool ids and index lists, bit for bit,
whatever the chunk size (ragged last chunks included).  The chunks select
rows of up to 40,960 pools in one pass (mini_prefill), wider rows from the
scoring pass's 64-pool group lists (mini_prefill_wide, 45,024 pools) or, past
65,536 pools, from sorted score tiles (mini_long); the unbounded calls use
the one-pass or tile selection."""
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


@pytest.mark.parametrize("name,chunk", [("mini_prefill", 64), ("mini_prefill", 50), ("mini_prefill", 200),
                                        ("mini_prefill", 1), ("mini_decode", 3), ("tiny", 10),
                                        ("mini_prefill_wide", 80), ("mini_prefill_wide", 40),
                                        ("mini_long", 2),
                                        pytest.param("prefill_4k_on_131k", 512, marks=pytest.mark.slow)])
def test_chunked_selection_matches_unbounded(harness, name, chunk):
    wl = syn.get(name)
    say(f"chunked selection {name} chunk={chunk}")
    dw = harness.DeviceWorkload(wl, prefill_chunk=chunk)
    dw.step_append()
    dw.step_scores()
    dw.step_select()
    torch.cuda.synchronize()
    ref = [dw.pool_ids.clone(), dw.indices.clone()]
    dw.pool_ids.fill_(0x5A5A5A5A)
    dw.indices.fill_(0x5A5A5A5A)
    dw.step_prefill_select()
    torch.cuda.synchronize()
    assert torch.equal(ref[0], dw.pool_ids)
    assert torch.equal(ref[1], dw.indices)
    n = dw.ws_chunk.numel()
    assert n <= chunk * dw.stride * 4 + (64 << 20), n          # bounded by the chunk, not by T
