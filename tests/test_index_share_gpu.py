"""IndexShare layer stacks on the GPU (through the C ABI) against the oracle.

Full layers (layer <= 1 or layer % 4 == 2; ik_llama_opt log, "GLM-5.2 DSA:
IndexShare") run the whole path and keep their index rows; shared layers
attend over the rows of the most recent full layer.  Seven layers of the
reduced batched-decode workload (fp16 index keys, one sink, 128-head MLA),
each with its own seeded inputs: layers 0, 1, 2 and 6 are full, 3-5 share
layer 2's selection.
"""

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O
from sparse_top_attention_indexer_amd import inputs
from test_parity_gpu import check_selection, dev, oracle_scores   # the suite's selection and score rules

pytestmark = pytest.mark.gpu
f64 = O.to_f64


@pytest.mark.parametrize("n", [3, 4])   # 3: token mode, MLA decode; 4: block mode (QSA), GQA prefill chunk
def test_layer_stack_shares_selections(n):
    wl = inputs.mini(n)
    n_layers = 7
    xs = [inputs.generate(wl, seed=4000 + il) for il in range(n_layers)]
    ds = [dev(x) for x in xs]
    keys = ("Q", "K", "V", "q_idx", "k_idx", "w", "k_scale")
    layers = [dict({k: d[k] for k in keys}, scale=wl.scale) for d in ds]
    outs, idxs = dsa.forward_layers(layers, wl.top_k, wl.c, ds[0]["q_pos"], n_sink=wl.n_sink,
                                    hadamard_q=wl.hadamard_q, kv_len=ds[0]["kv_len"])
    torch.cuda.synchronize()
    srcs = [dsa.index_share_source(il) for il in range(n_layers)]
    assert srcs == [O.index_share_source(il) for il in range(n_layers)] == [0, 1, 2, 2, 2, 2, 6]

    qp, kv = xs[0]["q_pos"].numpy(), xs[0]["kv_len"].numpy()
    rows = [(s, i) for s in range(wl.S) for i in range(0, wl.n_q, max(1, wl.n_q // 6))]   # a spread of rows
    ol = [dict({k: (None if x[k] is None else f64(x[k])) for k in keys}, scale=wl.scale) for x in xs]
    ref_outs, ref_idxs = O.forward_layers(ol, wl.top_k, wl.c, qp, kv, wl.n_sink if wl.c == 1 else 0,
                                          wl.hadamard_q, rows)
    worst_own, worst_ref = 0.0, 0.0
    for il in range(n_layers):
        got_idx = idxs[il].cpu().numpy().astype(np.int64)
        if srcs[il] != il:
            assert idxs[il] is idxs[srcs[il]]   # the source layer's rows, not a selection of its own
        else:
            pooled = O.block_pool(f64(xs[il]["k_idx"]), wl.c) if wl.c > 1 else None
            s_ref = oracle_scores(xs[il], wl, rows=rows, pooled=pooled)
            for s, i in rows:
                n_units = O.visible_tokens(int(qp[s, i]), int(kv[s])) // wl.c
                check_selection(got_idx[s, i], ref_idxs[il][s, i], s_ref[s, i], n_units, wl.k_out,
                                wl.n_sink if wl.c == 1 else 0)
        # the layer's attention over the rows it was given, against the oracle on the same rows
        want = O.sparse_attention(ol[il]["Q"], ol[il]["K"], ol[il]["V"], got_idx, qp, kv, wl.c, wl.scale, rows)
        got = outs[il].cpu().double().numpy()
        worst_own = max(worst_own, max(float(np.abs(got[s, i] - want[s, i]).max()) for s, i in rows))
        # and end to end where the selections agree
        same = [(s, i) for s, i in rows if np.array_equal(got_idx[s, i], ref_idxs[il][s, i])]
        for s, i in same:
            worst_ref = max(worst_ref, float(np.abs(got[s, i] - ref_outs[il][s, i]).max()))
    print(f"index share, {wl.name}, {n_layers} layers: |O - oracle(same rows)| {worst_own:.2e}, "
          f"|O - oracle stack| {worst_ref:.2e}")
    assert worst_own <= 2e-2 and worst_ref <= 2e-2


def test_shared_layer_differs_from_its_own_selection():
    # a shared layer really attends over its source's rows: with its own indexer
    # inputs it would select differently
    wl = inputs.mini(3)
    d2, d3 = dev(inputs.generate(wl, seed=4002)), dev(inputs.generate(wl, seed=4003))
    _, idx2 = dsa.forward(d2["Q"], d2["K"], d2["V"], d2["q_idx"], d2["k_idx"], d2["w"], wl.top_k, wl.c, d2["q_pos"],
                          k_scale=d2["k_scale"], n_sink=wl.n_sink, scale=wl.scale, kv_len=d2["kv_len"],
                          return_idx=True)
    _, idx3 = dsa.forward(d3["Q"], d3["K"], d3["V"], d3["q_idx"], d3["k_idx"], d3["w"], wl.top_k, wl.c, d3["q_pos"],
                          k_scale=d3["k_scale"], n_sink=wl.n_sink, scale=wl.scale, kv_len=d3["kv_len"],
                          return_idx=True)
    assert not torch.equal(idx2, idx3)
