"""Sparse attention over q8_0 latent rows (the quantised latent cache,
ik_llama_opt log, openPangu port, "Add OpenPangu q8_0 latent cache type"),
through the C ABI, against the CPU oracle.

The oracle attends over the exactly dequantised rows (oracle.decode_q8_0:
code x f16 scale), on the same selection the kernel gets.  The kernel rounds
each dequantised value to bf16 before the products, like a bf16 latent, so
the bar is the bf16 attention tolerance: 2e-2 absolute.  The distance to
attention over the unquantised bf16 rows is printed as a relative L-inf
(context: the page reports 0.0057 against an f16 cache), not gated.
"""

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O
from sparse_top_attention_indexer_amd import inputs
from test_parity_gpu import _oracle_idx, _rows_sample, dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
f64 = O.to_f64


def q8_latent(x):
    """(codes, scales) on the GPU, and the dequantised rows [S, n_kv, 1, 576] for the oracle."""
    codes, scales = inputs.q8_0_latent(x["K"].cpu())
    deq = O.decode_q8_0(codes.numpy()[:, :, 0, :], scales.view(torch.int16).numpy().view(np.uint16))
    return codes.to(DEV), scales.to(DEV), deq[:, :, None, :]


CASES = {
    "batched_decode_mini": lambda: inputs.mini(3),
    "long_decode_mini_outliers": lambda: inputs.mini(5),
    "prefill_mini": lambda: inputs.mini(2),
    "48_heads_split": lambda: inputs.Workload(
        "q8_48", 3, 2, 1500, 1400, 32, 128, torch.bfloat16, torch.bfloat16, "normal", 0.2, 900, 1, 1, False,
        "mla", 48, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=98),
    "block_mode": lambda: inputs.Workload(
        "q8_blk", 1, 60, 1000, 940, 16, 128, torch.bfloat16, torch.bfloat16, "normal", 0.25, 256, 16, 0, False,
        "mla", 128, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=99),
}


@pytest.mark.parametrize("case", list(CASES))
def test_q8_latent_attention_matches_oracle(case):
    wl = CASES[case]()
    x = inputs.generate(wl)
    idx, _ = _oracle_idx(x, wl)
    d = dev(x)
    codes, scales, deq = q8_latent(x)
    idx_d = torch.from_numpy(idx).to(torch.int32).to(DEV)
    got = dsa.sparse_attn(d["Q"], codes, codes[..., :512], d["q_pos"], idx_d, c=wl.c, kv_len=d["kv_len"],
                          scale=wl.scale, kv_scale=scales).cpu().double().numpy()
    rows = _rows_sample(wl, 16, seed=7)
    qp, kv = x["q_pos"].numpy(), x["kv_len"].numpy()
    ref = O.sparse_attention(f64(x["Q"]), deq, deq[..., :512], idx, qp, kv, wl.c, wl.scale, rows)
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    # context: distance to attention over the unquantised bf16 rows
    bf = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], idx_d, c=wl.c, kv_len=d["kv_len"],
                         scale=wl.scale).cpu().double().numpy()
    linf_rel = float(np.abs(got - bf).max() / np.abs(bf).max())
    print(f"{case}: max |O_q8 - oracle(dequantised)| {err:.2e}; relative L-inf to the bf16 rows {linf_rel:.4f}")
    assert err <= 2e-2


def test_q8_latent_dense_and_forward():
    # idx = NULL (dense causal over the q8 rows) and the whole path with a q8
    # latent: the selection is the indexer's (it does not read the latent), the
    # output the oracle's attention over the dequantised rows
    wl = inputs.mini(3)
    x = inputs.generate(wl)
    d = dev(x)
    codes, scales, deq = q8_latent(x)
    qp, kv = x["q_pos"].numpy(), x["kv_len"].numpy()
    dense = dsa.sparse_attn(d["Q"], codes, codes[..., :512], d["q_pos"], None, kv_len=d["kv_len"], scale=wl.scale,
                            kv_scale=scales).cpu().double().numpy()
    ref_dense = O.dense_attention(f64(x["Q"]), deq, deq[..., :512], qp, kv, wl.scale)
    assert float(np.abs(dense - ref_dense).max()) <= 2e-2
    o, idx = dsa.forward(d["Q"], codes, codes[..., :512], d["q_idx"], d["k_idx"], d["w"], wl.top_k, 1, d["q_pos"],
                         n_sink=wl.n_sink, scale=wl.scale, kv_len=d["kv_len"], kv_scale=scales, return_idx=True)
    o_bf, idx_bf = dsa.forward(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], d["w"], wl.top_k, 1, d["q_pos"],
                               n_sink=wl.n_sink, scale=wl.scale, kv_len=d["kv_len"], return_idx=True)
    assert torch.equal(idx, idx_bf)   # the selection does not depend on the latent's format
    ref = O.sparse_attention(f64(x["Q"]), deq, deq[..., :512], idx.cpu().numpy().astype(np.int64), qp, kv, 1,
                             wl.scale)
    err = float(np.abs(o.cpu().double().numpy() - ref).max())
    print(f"forward over q8 rows: max |O - oracle| {err:.2e}")
    assert err <= 2e-2
