"""dsa_topk_noalloc, the top-k entry point that allocates nothing, against
dsa_topk.

Two calls in a row through the C ABI on decode-shaped rows (the multi-block
path, whose histograms, counters and candidates live in the library's static
device scratch), the second with a smaller input: the scratch keeps the first
call's contents, so the second call shows that it clears what must start at
zero.  Each result must equal dsa_topk's on the same scores bit for bit (index
work).  A call whose workspace exceeds the scratch is refused on the host
before anything runs, and writes nothing.
"""

import ctypes

import pytest
import torch

import sparse_top_attention_indexer_amd as dsa

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKSPACE = -6


def decode_scores(S, n, seed):
    g = torch.Generator().manual_seed(seed)
    sc = torch.randn((S, 1, n), generator=g)
    sc[..., ::97] = torch.round(sc[..., ::97])   # some exact ties
    return sc.to(DEV)


def noalloc(sc, d, out):
    return dsa.lib().dsa_topk_noalloc(dsa._ptr(sc), ctypes.byref(d), dsa._ptr(out), dsa._stream())


def test_noalloc_topk_equals_topk_on_two_calls_then_refuses_oversize():
    # (S, units per row, top_k, sinks, seed): the long-decode shape, then a smaller one
    for S, n, k, sink, seed in [(8, 131072, 2048, 0, 1), (3, 40000, 1000, 1, 2)]:
        print(f"noalloc top-k: S={S} n_units={n} top_k={k} n_sink={sink}", flush=True)
        sc = decode_scores(S, n, seed)
        q_pos = torch.full((S, 1), n - 1, dtype=torch.int32, device=DEV)
        kv = torch.tensor([n - 37 * s for s in range(S)], dtype=torch.int32, device=DEV)
        d = dsa._topk_desc(S, 1, n, q_pos, kv, k, 1, sink)
        assert 0 < dsa.lib().dsa_topk_workspace_bytes(ctypes.byref(d)) <= (16 << 20)   # uses the scratch
        out = torch.full((S, 1, k), -7, dtype=torch.int32, device=DEV)
        assert noalloc(sc, d, out) == 0
        ref = dsa.topk(sc, q_pos, k, n_sink=sink, kv_len=kv)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    # 17 rows of 131072 units need more than the 16 MiB scratch: refused, untouched
    S, n, k = 17, 131072, 2048
    sc = decode_scores(S, n, 3)
    q_pos = torch.full((S, 1), n - 1, dtype=torch.int32, device=DEV)
    d = dsa._topk_desc(S, 1, n, q_pos, None, k, 1, 0)
    assert dsa.lib().dsa_topk_workspace_bytes(ctypes.byref(d)) > (16 << 20)
    out = torch.full((S, 1, k), -7, dtype=torch.int32, device=DEV)
    assert noalloc(sc, d, out) == WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == -7).all())
