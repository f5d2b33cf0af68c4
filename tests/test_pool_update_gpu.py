"""Incremental block pooling (dsa_block_pool_update, through the C ABI).

The pooled keys persist in a caller buffer across micro-batches; each call
re-pools only the blocks from a per-sequence first block up to the
sequence's complete blocks, and a sequence edit re-pools from its position on
(offgrid-sys llama-memory-hybrid-idx.h: persistent pooled keys, pools to
re-pool per micro-batch, stale position of an edit).  The bar: the buffer
after any series of updates equals the one-shot pool of the final keys bit
for bit, blocks outside every update keep their sentinel, and the one-shot
pool matches the float64 oracle.
"""

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O
from sparse_top_attention_indexer_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
C = 64
N_KV = 2085          # 32 complete blocks and a ragged tail
SENTINEL = -12345.0


def i32(v):
    return torch.tensor(v, dtype=torch.int32, device=DEV)


def test_micro_batches_then_edit_equal_one_shot():
    k = inputs.raw_key_batch(3, N_KV, seed=3001).to(DEV)
    nb = N_KV // C
    pooled = torch.full((3, nb, 128), SENTINEL, dtype=torch.float32, device=DEV)
    # three micro-batches with a different stored length per sequence; each
    # call re-pools from the first block the previous call left incomplete
    steps = [[700, 64, 0], [1500, 64, 1000], [N_KV, 2000, N_KV]]
    prev = [0, 0, 0]
    for kv in steps:
        dsa.block_pool_update(k, C, pooled, i32([p // C for p in prev]), kv_len=i32(kv))
        prev = kv
    final_blocks = [kv // C for kv in steps[-1]]
    ref = dsa.block_pool(k, C)
    torch.cuda.synchronize()
    for s in range(3):
        nbs = final_blocks[s]
        assert torch.equal(pooled[s, :nbs], ref[s, :nbs]), f"sequence {s}: incremental != one-shot"
        assert bool((pooled[s, nbs:] == SENTINEL).all()), f"sequence {s}: a block past the stored keys was written"
    # an edit of sequence 1 from position 1000 stales its pools from block 1000 // 64 on;
    # the other sequences ask for nothing (their first block is past their complete blocks)
    k[1, 1000:] = inputs.raw_key_batch(1, N_KV - 1000, seed=3002).to(DEV)[0]
    dsa.block_pool_update(k, C, pooled, i32([final_blocks[0], 1000 // C, final_blocks[2]]), kv_len=i32(steps[-1]))
    ref2 = dsa.block_pool(k, C)
    torch.cuda.synchronize()
    assert torch.equal(pooled[1, :final_blocks[1]], ref2[1, :final_blocks[1]])
    assert torch.equal(pooled[0], ref2[0]) and torch.equal(pooled[2], ref2[2])
    # and the one-shot pool against the float64 oracle (f32 sums of 64 bf16 rows)
    want = O.block_pool(O.to_f64(k.cpu()), C)
    assert np.allclose(ref2.cpu().double().numpy(), want, rtol=2e-6, atol=1e-6)


def test_update_without_lengths_covers_all_complete_blocks():
    k = inputs.raw_key_batch(2, N_KV, dtype=torch.float16, seed=3003).to(DEV)
    pooled = torch.full((2, N_KV // C, 128), SENTINEL, dtype=torch.float32, device=DEV)
    dsa.block_pool_update(k, C, pooled, i32([0, -5]))   # a negative first block counts as 0
    assert torch.equal(pooled, dsa.block_pool(k, C))
