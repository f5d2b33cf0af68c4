"""GQA attention over query tiles (attn_gqa_tile_kernel) against the oracle.

The tile kernel serves GQA calls in dense mode and in block mode with blocks
of a multiple of 32 tokens when a sequence holds 8 or more queries.  These
cases cover every head grouping it takes (1, 2, 4, 8, 16 heads per KV group),
ragged query tiles, key splits, block sizes 32 / 64 / 96 / 128, shortened
caches, rows that see nothing, shuffled lists with dead and repeated blocks,
and bf16 output.  Tolerance: 2e-2 absolute (bf16 attention).
"""

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def make(S, n_q, n_kv, Hq, Hkv, q_pos0, kv_len, seed):
    g = torch.Generator().manual_seed(seed)
    Q = torch.randn((S, n_q, Hq, 128), generator=g).to(torch.bfloat16)
    K = torch.randn((S, n_kv, Hkv, 128), generator=g).to(torch.bfloat16)
    V = torch.randn((S, n_kv, Hkv, 128), generator=g).to(torch.bfloat16)
    q_pos = (q_pos0 + torch.arange(n_q, dtype=torch.int32)).repeat(S, 1).contiguous()
    return Q, K, V, q_pos, torch.tensor(kv_len, dtype=torch.int32)


def block_lists(q_pos, kv_len, n_kv, c, k_out, seed, shuffle=True, repeats=True):
    """Per row k_out entries: distinct live blocks (0 <= b < n_cb) in random
    order, -1 where fewer exist; some rows list one block twice and carry
    dead entries (-1 and ids past n_cb) in between."""
    rng = np.random.default_rng(seed)
    S, n_q = q_pos.shape
    idx = np.full((S, n_q, k_out), -1, np.int32)
    for s in range(S):
        for i in range(n_q):
            n_vis = max(0, min(int(q_pos[s, i]) + 1, int(kv_len[s]), n_kv))
            n_cb = n_vis // c
            live = rng.permutation(n_cb)[:k_out] if shuffle else np.arange(min(n_cb, k_out))
            idx[s, i, :live.size] = live
            if repeats and live.size >= 3 and i % 3 == 0:
                idx[s, i, live.size - 1] = idx[s, i, 0]          # listed twice
            if live.size < k_out and i % 4 == 1:
                idx[s, i, live.size] = n_cb + 2                   # not a complete visible block: dead
            if live.size >= 2 and i % 5 == 2:
                idx[s, i, 1] = -1
    return idx


def run(Q, K, V, q_pos, kv_len, idx, c, scale, o_dtype=torch.float32):
    d = [t.to(DEV) for t in (Q, K, V, q_pos, kv_len)]
    idx_d = None if idx is None else torch.from_numpy(idx).to(DEV)
    return dsa.sparse_attn(d[0], d[1], d[2], d[3], idx_d, c=c, kv_len=d[4], scale=scale, o_dtype=o_dtype)


def oracle(Q, K, V, q_pos, kv_len, idx, c, scale):
    return O.sparse_attention(O.to_f64(Q), O.to_f64(K), O.to_f64(V), idx, q_pos.numpy(), kv_len.numpy(), c, scale)


TILE_CASES = {
    # name: (S, n_q, n_kv, Hq, Hkv, q_pos0, kv_len, c, k_out)
    "g8_c64_ragged_two_sequences": (2, 37, 2000, 32, 4, 1963, [2000, 1700], 64, 12),
    "g16_c32_one_tile": (1, 20, 1500, 32, 2, 1480, [1500], 32, 16),
    "g4_c96_two_tiles": (1, 70, 3000, 16, 4, 2930, [3000], 96, 10),
    "g2_c128_short_rows": (2, 9, 2500, 16, 8, 2491, [2500, 2100], 128, 6),
    "g1_c64_128_query_tile": (1, 130, 1200, 4, 4, 1070, [1200], 64, 8),
    "g8_c64_early_queries": (1, 40, 700, 32, 4, 0, [700], 64, 4),
}


@pytest.mark.parametrize("case", list(TILE_CASES))
def test_gqa_tiles_block_mode(case):
    S, n_q, n_kv, Hq, Hkv, q0, kv, c, k_out = TILE_CASES[case]
    Q, K, V, q_pos, kv_len = make(S, n_q, n_kv, Hq, Hkv, q0, kv, seed=100 + list(TILE_CASES).index(case))
    if n_q > 5:
        q_pos[0, 5] = -1   # a row that sees nothing
    idx = block_lists(q_pos.numpy(), kv, n_kv, c, k_out, seed=3)
    scale = 128 ** -0.5
    got = run(Q, K, V, q_pos, kv_len, idx, c, scale).cpu().double().numpy()
    ref = oracle(Q, K, V, q_pos, kv_len, idx, c, scale)
    err = float(np.abs(got - ref).max())
    print(f"{case}: max |O - oracle| {err:.2e}")
    assert err <= 2e-2
    if n_q > 5:
        assert np.all(got[0, 5] == 0.0)
    got16 = run(Q, K, V, q_pos, kv_len, idx, c, scale, torch.bfloat16).cpu().double().numpy()
    assert np.all(np.abs(got16 - ref) <= 2e-2 * np.maximum(1.0, np.abs(ref)))


@pytest.mark.parametrize("G,Hkv,n_q", [(8, 4, 45), (16, 1, 24), (2, 8, 100)])
def test_gqa_tiles_dense(G, Hkv, n_q):
    n_kv = 2200
    Q, K, V, q_pos, kv_len = make(2, n_q, n_kv, G * Hkv, Hkv, 2000, [2200, 2030], seed=11 + G)
    q_pos[1, 3] = -1
    q_pos[0, 7] = 5   # an early query inside a tile of late ones
    scale = 0.07
    got = run(Q, K, V, q_pos, kv_len, None, 1, scale).cpu().double().numpy()
    ref = oracle(Q, K, V, q_pos, kv_len, None, 1, scale)
    err = float(np.abs(got - ref).max())
    print(f"dense G={G} Hkv={Hkv} n_q={n_q}: max |O - oracle| {err:.2e}")
    assert err <= 2e-2
    assert np.all(got[1, 3] == 0.0)


def test_gqa_tiles_every_block_is_bitwise_dense():
    """A list naming every complete visible block, in any order, is the dense
    token set: the tile kernel sums in position order either way, so the rows
    agree bit for bit with the dense call."""
    S, n_q, n_kv, c = 2, 33, 1800, 64
    Q, K, V, q_pos, kv_len = make(S, n_q, n_kv, 32, 4, 1767, [1800, 1500], seed=5)
    k_out = n_kv // c
    dense = run(Q, K, V, q_pos, kv_len, None, 1, None)
    for shuffle in (False, True):
        idx = block_lists(q_pos.numpy(), [1800, 1500], n_kv, c, k_out, seed=9, shuffle=shuffle, repeats=False)
        # keep every live block: undo the dead entries the helper plants
        for s in range(S):
            for i in range(n_q):
                n_vis = max(0, min(int(q_pos[s, i]) + 1, int(kv_len[s])))
                n_cb = n_vis // c
                live = np.random.default_rng(i).permutation(n_cb) if shuffle else np.arange(n_cb)
                idx[s, i] = -1
                idx[s, i, :n_cb] = live
        got = run(Q, K, V, q_pos, kv_len, idx, c, None)
        assert torch.equal(got, dense)
