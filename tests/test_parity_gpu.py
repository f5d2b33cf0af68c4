"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances (the DSA targets; relative errors use the condition scale
sum_h |w| relu(q_h . k), which equals |s| for non-negative weights):
  indexer scores      1e-3 relative (f32 / bf16 / f16 keys), 2e-2 (fp8 keys,
                      against the scores of the dequantised keys)
  top-k on identical  bit-exact sets, ascending, -1 padded
  score inputs
  end-to-end sets     equal, except that an index may differ only when its
                      oracle score is within 1e-3 relative of the oracle's
                      k-th score
  attention           1e-4 absolute (f32), 2e-2 absolute (bf16), with the
                      oracle's selection fed to both sides
"""

import math

from dataclasses import replace

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O
from sparse_top_attention_indexer_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
f64 = O.to_f64


def dev(x):
    """GPU copies; an MLA value tensor stays a view of the latent rows it aliases."""
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items() if k != "V"}
    V = x["V"]
    if V.untyped_storage().data_ptr() == x["K"].untyped_storage().data_ptr():
        d["V"] = d["K"][..., :V.shape[-1]]
    else:
        d["V"] = V.to(DEV)
    return d


def rel_err(got, ref, cond):
    """Largest score error relative to the unit's condition scale; invisible
    units must agree exactly.

    cond(u) = sum_h |w_h| sum_d |q'_hd k_ud| is the scale of the sum of
    products that forms s(u) (cond_scale): a path that rounds the products or
    their sums in f32 is off by a small multiple of the unit roundoff times
    it, whatever the cancellation at the ReLU kink or between signed weights.
    The floor 1e-6 max_u cond(u) only guards rows whose every scale is zero."""
    inv = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inv), "visibility mismatch"
    worst = 0.0
    for gr, rr, cr, iv in zip(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]),
                              cond.reshape(-1, cond.shape[-1]), inv.reshape(-1, inv.shape[-1])):
        g, r, c = gr[~iv], rr[~iv], cr[~iv]
        if g.size == 0:
            continue
        worst = max(worst, float((np.abs(g - r) / (c + 1e-6 * c.max() + 1e-300)).max()))
    return worst


def cond_scale(x, wl, rows=None, pooled=None):
    """sum_h |w_h| sum_d |q'_hd k_ud| per (query, unit), q' the rotated query
    when the keys are stored rotated, k the dequantised key."""
    q = f64(x["q_idx"])
    if wl.hadamard_q:
        q = q @ O.hadamard(q.shape[-1]).T
    keys = np.abs(pooled if pooled is not None else f64(x["k_idx"]))
    ks = None if x.get("k_scale") is None or pooled is not None else np.abs(f64(x["k_scale"]))
    # with non-negative operands the ReLU is the identity, so the oracle's
    # score of |q'|, |k|, |w| is exactly the sum above
    return O.index_scores(np.abs(q), keys, np.abs(f64(x["w"])), x["q_pos"].cpu().numpy(),
                          x["kv_len"].cpu().numpy(), wl.c, ks, False, rows)


def oracle_scores(x, wl, rows=None, pooled=None):
    keys = pooled if pooled is not None else f64(x["k_idx"])
    ks = None if x.get("k_scale") is None or pooled is not None else f64(x["k_scale"])
    return O.index_scores(f64(x["q_idx"]), keys, f64(x["w"]), x["q_pos"].cpu().numpy(),
                          x["kv_len"].cpu().numpy(), wl.c, ks, wl.hadamard_q, rows)


def score_tol_tight(q_dtype, k_dtype, hadamard, H=64, D=128):
    """The score error each kernel path's arithmetic allows, relative to
    cond_scale, with margin.  (D + H) u (u = 2^-24) bounds f32 sums of D
    products and H weighted heads: 1.2e-5 at D = 128, H = 64.
      exact products (bf16 q and bf16 / f16 keys; f16 q and f16 keys; the
        f32 VALU path's fused products): 2e-5;
      a bf16 split of an operand (f32 pooled keys, a rotated or f16 q against
        bf16 keys): each operand exact to 2^-17, so 4e-5;
      q rounded to f16 once (fp8 keys, or a rotated / f32 q against f16
        keys): 2^-12 per product, so 3e-4."""
    mfma = D == 128 and H <= 64 and q_dtype in (torch.bfloat16, torch.float16)
    if not mfma:
        return 2e-5
    if k_dtype == torch.float8_e4m3fn:
        return 3e-4
    if k_dtype == torch.float16:
        return 2e-5 if (q_dtype in (torch.bfloat16, torch.float16) and not hadamard) else 3e-4
    if k_dtype == torch.bfloat16:
        return 2e-5 if (q_dtype == torch.bfloat16 and not hadamard) else 4e-5
    return 4e-5


def check_selection(got, ref, s_ref, n_vis, k_out, nf):
    """Set rule; returns True when the two selections are identical."""
    K = min(k_out, n_vis)
    live = got[got >= 0]
    assert live.size == K and np.all(got[K:] == -1), "dead slots must follow the live ones"
    assert np.all(np.diff(live) > 0), "ascending, unique"
    assert live.size == 0 or (live[0] >= 0 and live[-1] < n_vis), "only visible units"
    assert set(range(min(nf, n_vis))) <= set(live.tolist()), "forced sinks"
    rl = ref[ref >= 0]
    diff = set(live.tolist()) ^ set(rl.tolist())
    if not diff:
        return True
    rest = [j for j in rl.tolist() if j >= nf]
    s_k = min(s_ref[j] for j in rest)
    for j in diff:
        assert abs(s_ref[j] - s_k) <= 1e-3 * abs(s_k), f"unit {j}: {s_ref[j]} vs k-th {s_k}"
    return False


# ------------------------------------------------------------------ scores --

SCORE_CASES = {
    "tiny_f32_valu": lambda: inputs.preset(1),
    "prefill_bf16": lambda: inputs.mini(2),
    "decode_f16_keys": lambda: inputs.mini(3),
    "decode_fp8_hadamard": lambda: inputs.mini(5),
    "ragged_40_heads_f16_q": lambda: inputs.Workload(
        "ragged", 2, 37, 1001, 980, 40, 128, torch.float16, torch.bfloat16, "normal", 0.2, 128, 1, 0,
        False, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=77),
    "ragged_40_heads_f16_q_rows_of_4": lambda: inputs.Workload(
        "ragged4", 2, 36, 1001, 980, 40, 128, torch.float16, torch.bfloat16, "normal", 0.2, 128, 1, 0,
        False, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=80),
    "bf16_keys_hadamard_split_q": lambda: inputs.Workload(
        "had_bf16", 1, 20, 700, 690, 64, 128, torch.bfloat16, torch.bfloat16, "normal", 0.125, 64, 1, 0,
        True, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=78),
    "f32_keys_mfma": lambda: inputs.Workload(
        "f32k", 1, 9, 333, 320, 16, 128, torch.bfloat16, torch.float32, "normal", 0.25, 64, 1, 0,
        False, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=79),
    # f32 keys on the LDS-tiled kernel (rows in groups of 4): 64 heads (two
    # head blocks), and 40 heads with an f16 query split in two operands
    "f32_keys_tiled_64_heads": lambda: inputs.Workload(
        "f32kt", 2, 12, 1200, 1180, 64, 128, torch.bfloat16, torch.float32, "normal", 0.125, 64, 1, 0,
        False, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=82),
    "f32_keys_tiled_split_q": lambda: inputs.Workload(
        "f32kts", 1, 8, 700, 690, 40, 128, torch.float16, torch.float32, "normal", 0.2, 64, 1, 0,
        False, "gqa", 8, 1, 128, 128, torch.bfloat16, 0.1, seed=83),
}


@pytest.mark.parametrize("case", list(SCORE_CASES))
def test_index_scores_match_oracle(case):
    wl = SCORE_CASES[case]()
    x = inputs.generate(wl)
    if case.startswith("ragged_40_heads"):   # shorter caches and invisible queries
        x["kv_len"] = torch.tensor([1001, 640], dtype=torch.int32)
        x["q_pos"][0, 0] = -1
    d = dev(x)
    got = dsa.index_scores(d["q_idx"], d["k_idx"], d["w"], d["q_pos"], c=1, k_scale=d["k_scale"],
                           kv_len=d["kv_len"], hadamard_q=wl.hadamard_q).cpu().double().numpy()
    ref = oracle_scores(x, wl)
    cond = cond_scale(x, wl)
    tol = 2e-2 if wl.k_dtype == torch.float8_e4m3fn else 1e-3
    tight = score_tol_tight(wl.q_dtype, wl.k_dtype, wl.hadamard_q, wl.H, wl.D)
    err = rel_err(got, ref, cond)
    print(f"{case}: max relative score error {err:.2e} (tolerance {tol:g}, path bound {tight:g})")
    assert err <= tol
    assert err <= tight


def test_index_scores_on_pooled_blocks():
    wl = inputs.mini(4)
    x = inputs.generate(wl)
    pooled64 = O.block_pool(f64(x["k_idx"]), wl.c)
    pooled = torch.from_numpy(pooled64).to(torch.float32)
    got = dsa.index_scores(x["q_idx"].to(DEV), pooled.to(DEV), x["w"].to(DEV), x["q_pos"].to(DEV), c=wl.c,
                           kv_len=x["kv_len"].to(DEV)).cpu().double().numpy()
    p32 = pooled.double().numpy()
    ref = oracle_scores(x, wl, pooled=p32)
    cond = cond_scale(x, wl, pooled=p32)
    err = rel_err(got, ref, cond)
    tight = score_tol_tight(wl.q_dtype, torch.float32, False, wl.H, wl.D)
    print(f"pooled: max relative score error {err:.2e} (path bound {tight:g})")
    assert err <= 1e-3
    assert err <= tight


def test_block_pool_matches_oracle():
    g = torch.Generator().manual_seed(5)
    for dt, c, n_kv in [(torch.bfloat16, 64, 2000), (torch.float16, 16, 333), (torch.float32, 7, 100)]:
        k = torch.randn((2, n_kv, 128), generator=g).to(dt)
        got = dsa.block_pool(k.to(DEV), c).cpu().double().numpy()
        ref = O.block_pool(f64(k), c)
        assert got.shape == ref.shape
        assert np.allclose(got, ref, rtol=2e-6, atol=1e-6)


# ------------------------------------------------------------------- top-k --

def _topk_case(S, n_q, n_units, top_k, c=1, n_sink=0, kind="normal", q_pos=None, kv_len=None, seed=0):
    g = torch.Generator().manual_seed(seed)
    sc = torch.randn((S, n_q, n_units), generator=g)
    if kind == "ties":
        sc = torch.round(sc * 2)
    elif kind == "equal":
        sc = torch.zeros_like(sc)
    if q_pos is None:
        q_pos = torch.full((S, n_q), n_units * c - 1, dtype=torch.int32)
    kv = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    got = dsa.topk(sc.to(DEV), q_pos.to(DEV), top_k, c=c, n_sink=n_sink,
                   kv_len=None if kv is None else kv.to(DEV)).cpu().numpy()
    ref = O.topk(sc.double().numpy(), q_pos.numpy(), top_k // c,
                 None if kv is None else kv.numpy(), c, n_sink)
    assert np.array_equal(got, ref)


def test_topk_rows_in_lds_causal():
    n = 3000
    _topk_case(1, 300, n, 256, q_pos=torch.arange(n - 300, n, dtype=torch.int32)[None] - 700)
    # rows of every length on the long-row kernel (n_units > 2048): fewer keys
    # than top_k, then candidate counts below 512, 512..2048 and above 2048,
    # which load their keys 1, 4 and 16 at a time per thread; plain and tied
    q_pos = torch.arange(0, n, 47, dtype=torch.int32)[None]
    _topk_case(1, q_pos.shape[1], n, 100, q_pos=q_pos, n_sink=1, seed=14)
    _topk_case(1, q_pos.shape[1], n, 100, q_pos=q_pos, kind="ties", seed=15)


def test_topk_rows_in_lds_with_ties_and_sink():
    _topk_case(2, 40, 5000, 512, n_sink=3, kind="ties", seed=1)
    _topk_case(1, 8, 4000, 300, kind="equal", seed=2)


def test_topk_rows_in_registers_long_rows():
    """Rows of 4097..16384 units on the one-workgroup-per-row path (32 and 64
    keys per thread), causal positions, ties and sinks."""
    n = 6000
    _topk_case(1, 128, n, 700, q_pos=torch.arange(n - 128, n, dtype=torch.int32)[None] - 900, seed=11)
    _topk_case(1, 130, 12000, 1000, n_sink=2, kind="ties", seed=12)
    _topk_case(1, 128, 16384, 4096, kind="equal", seed=13)


def test_topk_multiblock_decode_rows():
    _topk_case(3, 1, 40000, 2048, n_sink=1, kv_len=[40000, 25000, 1000], seed=3)
    _topk_case(2, 1, 131072, 2048, seed=4)
    # a row length that is not a multiple of 4 (unaligned rows: per-unit loads), sinks
    _topk_case(2, 1, 40001, 2048, n_sink=2, kv_len=[40001, 39999], seed=19)


def test_topk_long_rows_thousand_rows():
    # 1000 rows of 16401 units (row starts not 16-byte aligned: per-unit
    # loads), ties: the long-row kernel, one workgroup per row
    _topk_case(1, 1000, 16401, 300, kind="ties", seed=21)


def test_topk_long_rows_many_rows():
    # more than 128 rows of more than 16384 units: one workgroup per row on the
    # long-row kernel (rows 16-byte aligned: float4 loads), causal lengths from
    # below top_k to the whole row, ties
    n = 20000
    q_pos = torch.arange(0, 130 * 150, 150, dtype=torch.int32)[None]
    _topk_case(1, 130, n, 1000, q_pos=q_pos, kind="ties", seed=20)


def test_topk_multiblock_ties_and_equal():
    _topk_case(2, 1, 50000, 1000, kind="ties", seed=5)
    _topk_case(1, 1, 30000, 999, kind="equal", seed=6)


@pytest.mark.parametrize("S,n_q,n,k,seed", [(1, 8, 1000, 100, 16), (1, 8, 5000, 700, 17), (2, 1, 40000, 2048, 18)])
def test_topk_signed_zero_ties(S, n_q, n, k, seed):
    # -0 and +0 are equal scores: they tie, and the tie goes to the lower
    # index.  About 98 % of the scores are zeros of random sign, so every row
    # cuts its tie at zero: the short- and long-row kernels and the
    # multi-block decode path
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((S, n_q, n), generator=g)
    sc = torch.where(x < 2.0, torch.zeros_like(x) * torch.sign(x), x)
    assert bool((torch.signbit(sc) & (sc == 0)).any()) and bool((~torch.signbit(sc) & (sc == 0)).any())
    q_pos = torch.full((S, n_q), n - 1, dtype=torch.int32)
    got = dsa.topk(sc.to(DEV), q_pos.to(DEV), k).cpu().numpy()
    ref = O.topk(sc.double().numpy(), q_pos.numpy(), k)
    assert np.array_equal(got, ref)


def test_topk_edge_rows():
    q_pos = torch.tensor([[-1, 0, 5, 63, 64, 1000]], dtype=torch.int32)
    _topk_case(1, 6, 1001, 64, n_sink=2, q_pos=q_pos, seed=7)
    _topk_case(1, 6, 1001, 4, n_sink=4, q_pos=q_pos, seed=8)      # every slot a sink
    _topk_case(1, 3, 125, 512, c=16, q_pos=torch.tensor([[15, 700, 1999]], dtype=torch.int32), seed=9)
    _topk_case(2, 1, 20000, 1, seed=10)                          # top-1 on long rows


# --------------------------------------------------------------- attention --

def _oracle_idx(x, wl):
    pooled = O.block_pool(f64(x["k_idx"]), wl.c) if wl.c > 1 else None
    s = oracle_scores(x, wl, pooled=pooled)
    return O.topk(s, x["q_pos"].numpy(), wl.k_out, x["kv_len"].numpy(), wl.c, wl.n_sink if wl.c == 1 else 0), s


def _rows_sample(wl, n=24, seed=0):
    rng = np.random.default_rng(seed)
    all_rows = [(s, i) for s in range(wl.S) for i in range(wl.n_q)]
    if len(all_rows) <= n:
        return all_rows
    pick = set(all_rows[:4] + all_rows[-4:])
    while len(pick) < n:
        pick.add(all_rows[int(rng.integers(len(all_rows)))])
    return sorted(pick)


def _attn_tol(wl):
    return 1e-4 if wl.a_dtype == torch.float32 else 2e-2


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_sparse_attention_matches_oracle_on_oracle_selection(n):
    wl = inputs.mini(n)
    x = inputs.generate(wl)
    idx, _ = _oracle_idx(x, wl)
    d = dev(x)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx).to(torch.int32).to(DEV),
                          c=wl.c, kv_len=d["kv_len"], scale=wl.scale).cpu().double().numpy()
    rows = _rows_sample(wl)
    ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, x["q_pos"].numpy(),
                             x["kv_len"].numpy(), wl.c, wl.scale, rows)
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    print(f"config {n} mini: max |O - oracle| {err:.2e} over {len(rows)} rows")
    assert err <= _attn_tol(wl)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_dense_attention_matches_oracle(n):
    wl = inputs.mini(n)
    x = inputs.generate(wl)
    d = dev(x)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], None, kv_len=d["kv_len"],
                          scale=wl.scale).cpu().double().numpy()
    rows = _rows_sample(wl, 12, seed=1)
    ref = O.dense_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), x["q_pos"].numpy(), x["kv_len"].numpy(),
                            wl.scale, rows)
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    assert err <= _attn_tol(wl)


def test_gqa_token_mode_uneven_groups_split_streams():
    """GQA in token mode: 6 KV groups (the second workgroup row has waves
    without a group), 4 heads per group (MFMA columns padded to 16), lists
    with dead entries, streams split over several workgroups, f32 and bf16
    output."""
    bf = torch.bfloat16
    wl = inputs.Workload("gqa6", 2, 5, 3000, 2990, 16, 128, bf, bf, "normal", 0.25, 700, 1, 0,
                         False, "gqa", 24, 6, 128, 128, bf, 128 ** -0.5, seed=81)
    x = inputs.generate(wl)
    x["kv_len"] = torch.tensor([3000, 2500], dtype=torch.int32)
    idx, _ = _oracle_idx(x, wl)
    idx[0, 1, ::7] = -1
    idx[1, 3, 100:200] = -1
    d = dev(x)
    idx_d = torch.from_numpy(idx).to(torch.int32).to(DEV)
    rows = [(s, i) for s in range(wl.S) for i in range(wl.n_q)]
    ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, x["q_pos"].numpy(),
                             x["kv_len"].numpy(), 1, wl.scale, rows)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], idx_d, kv_len=d["kv_len"],
                          scale=wl.scale).cpu().double().numpy()
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    print(f"gqa token mode: max |O - oracle| {err:.2e}")
    assert err <= 2e-2
    got16 = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], idx_d, kv_len=d["kv_len"],
                            scale=wl.scale, o_dtype=torch.bfloat16).cpu().double().numpy()
    for s, i in rows:
        r = ref[s, i]
        assert np.all(np.abs(got16[s, i] - r) <= 2e-2 * np.maximum(1.0, np.abs(r)))


MLA_SHAPE_CASES = {
    # 48 heads: waves 3..7 of the workgroup hold no heads; decode-like rows
    # with a split stream
    "mla_48_heads_split": lambda: inputs.Workload(
        "mla48", 3, 2, 1500, 1400, 32, 128, torch.bfloat16, torch.bfloat16, "normal", 0.2, 900, 1, 1, False,
        "mla", 48, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=94),
    # 144 heads: a second row of workgroups with one wave of heads
    "mla_144_heads": lambda: inputs.Workload(
        "mla144", 1, 40, 700, 660, 32, 128, torch.bfloat16, torch.bfloat16, "normal", 0.2, 300, 1, 0, False,
        "mla", 144, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=95),
    # decode rows that take workgroups of 64 heads (waves 0, 1, 6, 7 hold the
    # heads, the other four only gather): one head group, and three
    "mla_64_heads_decode": lambda: inputs.Workload(
        "mla64", 5, 1, 3001, 3000, 32, 128, torch.bfloat16, torch.bfloat16, "normal", 0.2, 1024, 1, 1, False,
        "mla", 64, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=97),
    "mla_192_heads_decode": lambda: inputs.Workload(
        "mla192", 3, 1, 2500, 2499, 32, 128, torch.bfloat16, torch.bfloat16, "normal", 0.2, 1024, 1, 0, False,
        "mla", 192, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=98),
    # block mode: 16-token blocks plus the tail
    "mla_block_mode": lambda: inputs.Workload(
        "mlablk", 1, 60, 1000, 940, 16, 128, torch.bfloat16, torch.bfloat16, "normal", 0.25, 256, 16, 0, False,
        "mla", 128, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=96),
}


@pytest.mark.parametrize("case", list(MLA_SHAPE_CASES))
def test_mla_head_counts_and_block_mode(case):
    wl = MLA_SHAPE_CASES[case]()
    x = inputs.generate(wl)
    idx, _ = _oracle_idx(x, wl)
    d = dev(x)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx).to(torch.int32).to(DEV),
                          c=wl.c, kv_len=d["kv_len"], scale=wl.scale).cpu().double().numpy()
    rows = _rows_sample(wl, 16, seed=3)
    ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, x["q_pos"].numpy(),
                             x["kv_len"].numpy(), wl.c, wl.scale, rows)
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    print(f"{case}: max |O - oracle| {err:.2e} over {len(rows)} rows")
    assert err <= 2e-2


@pytest.mark.parametrize("case", ["mla_48_heads_split", "mla_144_heads", "mla_64_heads_decode",
                                  "mla_192_heads_decode"])
def test_mla_writes_only_its_output(case):
    # Waves without heads (48 heads: waves 3..7 of every workgroup; 144: waves
    # 1..7 of the second head block) run their products on head 0's query and
    # must write nothing.  The output sits inside a NaN-filled buffer whose
    # margins (as long as a whole row of 128 heads) must come back untouched;
    # every output element must be written, with the bits of a plain call.
    wl = MLA_SHAPE_CASES[case]()
    x = inputs.generate(wl)
    idx, _ = _oracle_idx(x, wl)
    d = dev(x)
    idx_d = torch.from_numpy(idx).to(torch.int32).to(DEV)
    kw = dict(c=wl.c, kv_len=d["kv_len"], scale=wl.scale)
    plain = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], idx_d, **kw)
    n, margin = plain.numel(), 128 * 512
    buf = torch.full((n + 2 * margin,), float("nan"), dtype=torch.float32, device=DEV)
    out = buf[margin:margin + n].view(plain.shape)
    dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], idx_d, out=out, **kw)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.isnan(b[:margin]).all() and torch.isnan(b[margin + n:]).all()
    got = b[margin:margin + n]
    assert not torch.isnan(got).any()
    assert torch.equal(got.view(torch.int32), plain.cpu().reshape(-1).view(torch.int32))


def test_mla_long_token_lists_and_trimmed_tails():
    # Token lists of 3000 entries, longer than the 2048 the MLA prologue
    # fetches up front, on one stream per row (130 rows: no split).  The live
    # entries end before 1024, between 1024 and 2048, or past 2048, and a dead
    # (-1) and an invisible id sit inside every list: the trim of the trailing
    # dead entries past the prefetched window, and the token ring refills.
    wl = inputs.Workload("mla_long_list", 1, 130, 4000, 3870, 32, 128, torch.bfloat16, torch.bfloat16, "normal",
                         0.2, 2048, 1, 0, False, "mla", 128, 1, 576, 512, torch.bfloat16, 576 ** -0.5, seed=97)
    x = inputs.generate(wl)
    k_sel, ends = 3000, [700, 1500, 2600, 3000]
    g = np.random.default_rng(97)
    qp = x["q_pos"].numpy()
    idx = np.full((1, wl.n_q, k_sel), -1, dtype=np.int32)
    for i in range(wl.n_q):
        n_vis, live = int(qp[0, i]) + 1, ends[i % 4]
        idx[0, i, :live] = g.permutation(n_vis)[:live]
        idx[0, i, 3] = -1
        idx[0, i, 7] = n_vis + 5 if n_vis + 5 < wl.n_kv else -1   # a key after the query
    d = dev(x)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx).to(DEV), kv_len=d["kv_len"],
                          scale=wl.scale).cpu().double().numpy()
    rows = [(0, i) for i in (0, 1, 2, 3, 64, 65, 66, 67, 126, 127, 128, 129)]
    ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, qp, x["kv_len"].numpy(), 1, wl.scale,
                             rows)
    err = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    print(f"long token lists: max |O - oracle| {err:.2e} over {len(rows)} rows")
    assert err <= 2e-2


def test_attention_bf16_output_and_empty_rows():
    wl = inputs.mini(2)
    x = inputs.generate(wl)
    x["q_pos"][0, :3] = -1
    idx, _ = _oracle_idx(x, wl)
    d = dev(x)
    got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx).to(torch.int32).to(DEV),
                          scale=wl.scale, o_dtype=torch.bfloat16).cpu()
    assert got.dtype == torch.bfloat16
    assert torch.count_nonzero(got[0, :3]) == 0 and not torch.isnan(got).any()
    rows = [(0, 5), (0, 400), (0, 699)]
    ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, x["q_pos"].numpy(), None, 1,
                             wl.scale, rows)
    for s, i in rows:
        r = ref[s, i]
        assert np.all(np.abs(got[s, i].double().numpy() - r) <= 2e-2 * np.maximum(1.0, np.abs(r)))


# ------------------------------------------------------------ invariants --

EXACT_DENSE = {
    "f32": lambda: inputs.preset(1),
    "mla_prefill": lambda: inputs.Workload("mla_small", 1, 300, 300, 0, 64, 128, torch.bfloat16, torch.bfloat16,
                                           "normal", 0.125, 512, 1, 0, False, "mla", 128, 1, 576, 512,
                                           torch.bfloat16, 1 / 24, seed=90),
    "mla_decode_split": lambda: inputs.Workload("mla_dec", 3, 1, 1500, 1499, 64, 128, torch.bfloat16,
                                                torch.float16, "normal", 0.125, 2048, 1, 1, False, "mla",
                                                128, 1, 576, 512, torch.bfloat16, 1 / 24, seed=91),
    "gqa": lambda: inputs.Workload("gqa_small", 1, 200, 200, 0, 16, 128, torch.bfloat16, torch.bfloat16,
                                   "normal", 0.25, 256, 1, 0, False, "gqa", 32, 4, 128, 128, torch.bfloat16,
                                   1 / math.sqrt(128), seed=92),
}


@pytest.mark.parametrize("case", list(EXACT_DENSE))
def test_sparse_is_bitwise_dense_when_topk_covers_all_keys(case):
    """top_k >= n_kv: the indexer is an exact no-op (ik_llama.cpp PR #2058, first commit)."""
    wl = EXACT_DENSE[case]()
    wl = inputs.replace(wl, top_k=max(wl.top_k, wl.n_kv))
    x = dev(inputs.generate(wl))
    o_sparse = dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, 1, x["q_pos"],
                           k_scale=x["k_scale"], n_sink=wl.n_sink, scale=wl.scale, kv_len=x["kv_len"])
    o_dense = dsa.sparse_attn(x["Q"], x["K"], x["V"], x["q_pos"], None, kv_len=x["kv_len"], scale=wl.scale)
    assert torch.equal(o_sparse, o_dense)


def test_block_mode_dense_below_threshold_and_cuts_on_blocks():
    """Block selection is dense below top_k + c - 1 tokens and whole blocks
    otherwise (llama.cpp mirror commit c88c916636, first and third paragraphs)."""
    c, top_k = 16, 128
    wl = inputs.Workload("blk", 1, 300, 300, 0, 16, 128, torch.bfloat16, torch.bfloat16, "normal", 0.25, top_k,
                         c, 0, False, "gqa", 32, 4, 128, 128, torch.bfloat16, 1 / math.sqrt(128), seed=93)
    x = dev(inputs.generate(wl))
    o, idx = dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], top_k, c, x["q_pos"],
                         scale=wl.scale, return_idx=True)
    o_dense = dsa.sparse_attn(x["Q"], x["K"], x["V"], x["q_pos"], None, scale=wl.scale)
    idx = idx.cpu().numpy()
    thr = top_k + c - 1
    for i in range(wl.n_q):
        n_vis = i + 1
        live = idx[0, i][idx[0, i] >= 0]
        if n_vis <= thr:
            assert live.tolist() == list(range(n_vis // c))
            # same tokens in the same order; the split of the stream may differ
            assert torch.allclose(o[0, i], o_dense[0, i], atol=2e-3, rtol=0)
        else:
            assert live.size == top_k // c
    assert not torch.isnan(o).any()


def test_forward_is_deterministic():
    wl = inputs.mini(3)
    x = dev(inputs.generate(wl))
    a = dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, 1, x["q_pos"],
                    k_scale=x["k_scale"], n_sink=wl.n_sink, return_idx=True, return_scores=True)
    b = dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, 1, x["q_pos"],
                    k_scale=x["k_scale"], n_sink=wl.n_sink, return_idx=True, return_scores=True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_sequences_are_independent():
    """n_seq sequences in one call give the same rows as each alone (PR #2058, UPDATE 5)."""
    wl = inputs.mini(3)
    x = dev(inputs.generate(wl))
    kw = dict(k_scale=None, n_sink=wl.n_sink, return_idx=True)
    o_all, i_all = dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, 1, x["q_pos"], **kw)
    for s in (0, wl.S - 1):
        sl = slice(s, s + 1)
        o1, i1 = dsa.forward(x["Q"][sl], x["K"][sl], x["V"][sl], x["q_idx"][sl], x["k_idx"][sl], x["w"][sl],
                             wl.top_k, 1, x["q_pos"][sl].contiguous(), **kw)
        assert torch.equal(i1[0], i_all[s])
        assert torch.allclose(o1[0], o_all[s], atol=1e-6, rtol=0)


# ------------------------------------------------------------- end to end --

def _end_to_end(wl, x, d, rows):
    o, idx, scores = dsa.forward(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], d["w"], wl.top_k, wl.c,
                                 d["q_pos"], k_scale=d["k_scale"], n_sink=wl.n_sink if wl.c == 1 else 0,
                                 scale=wl.scale, hadamard_q=wl.hadamard_q, kv_len=d["kv_len"],
                                 return_idx=True, return_scores=True)
    torch.cuda.synchronize()
    qp = x["q_pos"].cpu().numpy()
    kv = x["kv_len"].cpu().numpy()
    pooled = O.block_pool(f64(x["k_idx"]), wl.c) if wl.c > 1 else None
    ref_s = oracle_scores(x, wl, rows=rows, pooled=pooled)
    cond = cond_scale(x, wl, rows=rows, pooled=pooled)
    ref_idx = O.topk(ref_s, qp, wl.k_out, kv, wl.c, wl.n_sink if wl.c == 1 else 0, rows)
    got_s = scores.cpu().double().numpy()
    got_idx = idx.cpu().numpy().astype(np.int64)
    tol_s = 2e-2 if wl.k_dtype == torch.float8_e4m3fn else 1e-3
    tight_s = score_tol_tight(wl.q_dtype, torch.float32 if wl.c > 1 else wl.k_dtype, wl.hadamard_q, wl.H, wl.D)
    if wl.c > 1:   # the library's pooled keys are f32 sums of c rows: c u of the rows' magnitude more
        tight_s = max(tight_s, 1e-4)
    worst_s, same, worst_o, worst_a = 0.0, 0, 0.0, 0.0
    ref_o = O.sparse_attention(arr(x["Q"]), arr(x["K"]), arr(x["V"]), ref_idx, qp, kv, wl.c, wl.scale, rows)
    got_o = o.cpu().double().numpy()
    # the attention kernel on the oracle's own selection (identical inputs on both sides)
    oidx = torch.full(idx.shape, -1, dtype=torch.int32)
    for s, i in rows:
        oidx[s, i] = torch.from_numpy(ref_idx[s, i].astype(np.int32))
    o_on_ref = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], oidx.to(DEV), c=wl.c, kv_len=d["kv_len"],
                               scale=wl.scale).cpu().double().numpy()
    for s, i in rows:
        n_vis = O.visible_tokens(int(qp[s, i]), int(kv[s]))
        n_units = n_vis // wl.c
        worst_s = max(worst_s, rel_err(got_s[s, i, :n_units], ref_s[s, i, :n_units], cond[s, i, :n_units]))
        ident = check_selection(got_idx[s, i], ref_idx[s, i], ref_s[s, i], n_units, wl.k_out,
                                wl.n_sink if wl.c == 1 else 0)
        worst_a = max(worst_a, float(np.abs(o_on_ref[s, i] - ref_o[s, i]).max()))
        if ident:
            same += 1
            worst_o = max(worst_o, float(np.abs(got_o[s, i] - ref_o[s, i]).max()))
    print(f"{wl.name}: rows {len(rows)}, identical sets {same} (others differ only at near-ties), "
          f"score err {worst_s:.2e}, |O(oracle sel) - oracle| {worst_a:.2e}, |O - oracle| {worst_o:.2e}")
    assert worst_s <= tol_s
    assert worst_s <= tight_s, f"score error {worst_s:.2e} above the path bound {tight_s:g}"
    assert worst_a <= _attn_tol(wl)
    assert worst_o <= _attn_tol(wl)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_forward_matches_oracle_small(n):
    wl = inputs.mini(n)
    x = inputs.generate(wl)
    _end_to_end(wl, x, dev(x), _rows_sample(wl, 32, seed=n))


DECODE_STREAM_CASES = {
    # few long rows: the scores go through the decode stream kernel and its
    # fused histogram (f16 and bf16 keys; fp8 keys are the long-decode mini)
    "f16_keys_ragged": lambda: replace(inputs.mini(3), name="dec_f16", S=3, n_kv=7001, q_pos0=7000, seed=91),
    "bf16_keys_ragged": lambda: replace(inputs.mini(3), name="dec_bf16", S=2, n_kv=6500, q_pos0=6499,
                                        k_dtype=torch.bfloat16, seed=92),
    # f32 token keys on rows longer than 16384 units: the generic MFMA score
    # kernel (keys split into two bf16 operands) feeding the fused histogram
    "f32_keys_long_rows_generic_kernel_hist": lambda: replace(
        inputs.mini(3), name="dec_f32", S=2, n_kv=20000, q_pos0=19999, k_dtype=torch.float32, top_k=1024, seed=93),
}


@pytest.mark.parametrize("case", list(DECODE_STREAM_CASES))
def test_forward_decode_stream_matches_oracle(case):
    wl = DECODE_STREAM_CASES[case]()
    x = inputs.generate(wl)
    x["kv_len"] = torch.tensor([wl.n_kv - 37 * s for s in range(wl.S)], dtype=torch.int32)
    _end_to_end(wl, x, dev(x), [(s, 0) for s in range(wl.S)])


PREP_CASES = {
    # every operand form of the decode stream kernel's prepared queries:
    # bf16 q used as it is, bf16 q rotated and split into two bf16 operands,
    # f16 q prescaled for f16 keys, rotated bf16 / f16 q prescaled for fp8
    # keys, one and two blocks of 32 heads (24 heads: the second half padded)
    "bf16_q_bf16_keys": dict(k_dtype=torch.bfloat16, hadamard_q=False),
    "bf16_q_bf16_keys_rotated_split": dict(k_dtype=torch.bfloat16, hadamard_q=True),
    "bf16_q_f16_keys": dict(k_dtype=torch.float16, hadamard_q=False),
    "bf16_q_fp8_keys_rotated": dict(k_dtype=torch.float8_e4m3fn, hadamard_q=True),
    "f16_q_fp8_keys_rotated_24_heads": dict(k_dtype=torch.float8_e4m3fn, hadamard_q=True, q_dtype=torch.float16, H=24),
    "f16_q_bf16_keys_48_heads": dict(k_dtype=torch.bfloat16, hadamard_q=False, q_dtype=torch.float16, H=48),
}


@pytest.mark.parametrize("case", list(PREP_CASES))
def test_decode_stream_scores_bitwise_standalone(case):
    """Decode rows score through score_prep_kernel's operands and the stream
    kernel; the standalone call converts the same query in every wave of the
    generic MFMA kernel, with the same products in the same order.  The two
    score rows must agree bit for bit (the prep kernel's conversion is
    query_operands' arithmetic, reordered only across lanes)."""
    wl = replace(inputs.mini(3), name="prep_" + case, S=3, n_kv=9001, q_pos0=9000, seed=97, **PREP_CASES[case])
    x = inputs.generate(wl)
    d = dev(x)
    _, _, scores = dsa.forward(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], d["w"], wl.top_k, wl.c, d["q_pos"],
                               k_scale=d["k_scale"], n_sink=wl.n_sink, scale=wl.scale, hadamard_q=wl.hadamard_q,
                               kv_len=d["kv_len"], return_idx=True, return_scores=True)
    alone = dsa.index_scores(d["q_idx"], d["k_idx"], d["w"], d["q_pos"], k_scale=d["k_scale"], kv_len=d["kv_len"],
                             hadamard_q=wl.hadamard_q)
    torch.cuda.synchronize()
    n_vis = int(x["kv_len"].min())
    a = scores[..., :n_vis].contiguous().view(torch.int32)
    b = alone[..., :n_vis].contiguous().view(torch.int32)
    assert torch.equal(a, b), f"{case}: {int((a != b).sum())} scores differ"


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_forward_matches_oracle_full_size_sampled(n):
    """The full-size workloads, in the launch configuration the benchmark times,
    checked on sampled rows."""
    wl = inputs.preset(n)
    d = inputs.generate(wl, device=DEV)
    rows = _rows_sample(wl, 20 if wl.n_q > 1 else wl.S, seed=10 + n)
    # and the rows at the dense threshold: visible length top_k (+ c - 1 in block mode) -1 .. +2
    qp_all = d["q_pos"].cpu().numpy()
    thr = wl.top_k + (wl.c - 1 if wl.c > 1 else 0)
    edge = [(s, i) for s in range(wl.S) for i in range(wl.n_q) if thr - 1 <= qp_all[s, i] + 1 <= thr + 2]
    rows = sorted(set(rows) | set(edge[:8]))
    # the oracle gets CPU copies of what the sampled rows read; the attention
    # rows move to the host only when the oracle indexes them
    x = {"q_pos": d["q_pos"].cpu(), "kv_len": d["kv_len"].cpu(), "w": d["w"].cpu(), "q_idx": d["q_idx"].cpu(),
         "k_idx": d["k_idx"].cpu(), "k_scale": None if d["k_scale"] is None else d["k_scale"].cpu(),
         "Q": _Lazy(d["Q"]), "K": _Lazy(d["K"]), "V": _Lazy(d["V"])}
    _end_to_end(wl, x, d, rows)


class _Lazy:
    """[S, n, H, D] GPU tensor seen by the oracle: x[s, i] is one row, x[s] a sequence."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return f64(self.t[key])
        return _LazySeq(self.t[key])


class _LazySeq:
    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        tok = torch.from_numpy(np.asarray(key[0], dtype=np.int64)).to(self.t.device)
        return f64(self.t[tok][(slice(None),) + tuple(key[1:])])


def arr(t):
    return f64(t) if isinstance(t, torch.Tensor) else t


def test_gqa_block_mode_list_order_repeats_and_dead_rows():
    # block mode with blocks of 64 and 8 heads per KV group: two sequences (one
    # with fewer stored keys), 44 rows, one row that sees nothing, and a second
    # index list with every row's blocks shuffled, one block listed twice (it
    # is attended once per listing) and -1 entries mixed in.
    wl = replace(inputs.mini(4), name="qsa_tiles", S=2, n_q=44, n_kv=3000, q_pos0=2956, c=64, top_k=640)
    x = inputs.generate(wl)
    x["kv_len"] = torch.tensor([3000, 2600], dtype=torch.int32)
    x["q_pos"][1, 5] = -1
    d = dev(x)
    qp, kv = x["q_pos"].numpy(), x["kv_len"].numpy()
    ref_idx, _ = _oracle_idx(x, wl)
    rng = np.random.default_rng(7)
    mixed = ref_idx.copy()
    for s in range(wl.S):
        for i in range(wl.n_q):
            row = mixed[s, i]
            live = row[row >= 0]
            if live.size >= 2:
                perm = rng.permutation(live)
                perm[-1] = perm[0]   # one block listed twice (the last distinct one dropped)
                row[:] = -1
                start = 1 if live.size < row.size else 0   # a -1 in front where the row has room
                row[start:start + live.size] = perm
    rows = [(s, i) for s in range(wl.S) for i in range(wl.n_q)]
    worst = 0.0
    for idx in (ref_idx, mixed):
        got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx.astype(np.int32)).to(DEV),
                              c=wl.c, kv_len=d["kv_len"], scale=wl.scale).cpu().double().numpy()
        ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, qp, kv, wl.c, wl.scale)
        worst = max(worst, float(np.abs(got - ref).max()))
        assert np.all(got[1, 5] == 0.0)
    print(f"gqa block mode, shuffled and repeated lists: max |O - oracle| {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("c", [32, 96, 128])
def test_gqa_query_tiles_block_sizes(c):
    # the query-tile GQA kernel at block sizes of 1, 3 and 4 key tiles: with
    # blocks of one tile the two tiles of a step belong to different blocks
    # (different multiplicities per query); with three the block of a tile
    # comes from the multiply-high division.  37 rows (ragged query tiles),
    # two sequences with different stored lengths, and lists with every row's
    # blocks shuffled and one block listed twice.
    wl = replace(inputs.mini(4), name="qsa_tiles_c", S=2, n_q=37, n_kv=3000, q_pos0=2963, c=c, top_k=10 * c)
    x = inputs.generate(wl, seed=200 + c)
    x["kv_len"] = torch.tensor([3000, 2700], dtype=torch.int32)
    d = dev(x)
    qp, kv = x["q_pos"].numpy(), x["kv_len"].numpy()
    ref_idx, _ = _oracle_idx(x, wl)
    rng = np.random.default_rng(c)
    mixed = ref_idx.copy()
    for s in range(wl.S):
        for i in range(wl.n_q):
            row = mixed[s, i]
            live = row[row >= 0]
            if live.size >= 2:
                perm = rng.permutation(live)
                perm[-1] = perm[0]
                row[:] = -1
                row[:live.size] = perm
    worst = 0.0
    for idx in (ref_idx, mixed):
        got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"], torch.from_numpy(idx.astype(np.int32)).to(DEV),
                              c=wl.c, kv_len=d["kv_len"], scale=wl.scale).cpu().double().numpy()
        ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), idx, qp, kv, wl.c, wl.scale)
        worst = max(worst, float(np.abs(got - ref).max()))
    print(f"gqa query tiles, blocks of {c}: max |O - oracle| {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (16, 1)])
def test_gqa_query_tiles_group_sizes(hq, hkv):
    # the query-tile GQA kernel at 1, 2, 4 and 16 heads per KV group (256, 128,
    # 64 and 16 queries a workgroup), dense and in block mode with random
    # block lists: ragged query tiles, two sequences of different stored
    # lengths, and ~45 pairs of key tiles a workgroup, so that the LDS ring of
    # four pairs is reused many times while the waves run at their own pace.
    wl = replace(inputs.mini(4), name="qsa_groups", S=2, n_q=300, n_kv=2900, q_pos0=2600, c=64, top_k=16 * 64,
                 Hq=hq, Hkv=hkv)
    x = inputs.generate(wl, seed=300 + 10 * hq + hkv)
    x["kv_len"] = torch.tensor([2900, 2750], dtype=torch.int32)
    d = dev(x)
    qp, kv = x["q_pos"].numpy(), x["kv_len"].numpy()
    rng = np.random.default_rng(10 * hq + hkv)
    idx = np.full((wl.S, wl.n_q, 16), -1, np.int64)
    for s in range(wl.S):
        for i in range(wl.n_q):
            n_cb = O.visible_tokens(int(qp[s, i]), int(kv[s])) // wl.c
            pick = rng.choice(n_cb, size=min(15, n_cb), replace=False)
            idx[s, i, 1:1 + pick.size] = pick
    rows = _rows_sample(wl, n=40, seed=hq + hkv)
    worst = {}
    for name, sel in (("dense", None), ("blocks", idx)):
        got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"],
                              None if sel is None else torch.from_numpy(sel.astype(np.int32)).to(DEV),
                              c=wl.c, kv_len=d["kv_len"], scale=wl.scale).cpu().double().numpy()
        ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), sel, qp, kv, wl.c, wl.scale, rows=rows)
        worst[name] = max(float(np.abs(got[s, i] - ref[s, i]).max()) for s, i in rows)
    print(f"gqa query tiles, {hq // hkv} heads a group: max |O - oracle| {worst}")
    assert max(worst.values()) <= 2e-2


@pytest.mark.parametrize("n_kv", [20, 40, 100])
def test_gqa_query_tiles_short_streams(n_kv):
    # the query-tile GQA kernel on streams of one to four key tiles (one or
    # two pairs: the ring never wraps, and an odd tile count leaves the last
    # pair half empty), dense and in block mode, with causal queries from
    # position 0; one sequence's block lists are all dead, so its queries
    # attend to their incomplete tails only.
    wl = replace(inputs.mini(4), name="qsa_short", S=2, n_q=40, n_kv=n_kv, q_pos0=0, c=32, top_k=4 * 32)
    x = inputs.generate(wl, seed=400 + n_kv)
    d = dev(x)
    qp = x["q_pos"].numpy()
    kv = np.full(wl.S, n_kv, np.int64)
    idx = np.full((wl.S, wl.n_q, 4), -1, np.int64)
    rng = np.random.default_rng(n_kv)
    for i in range(wl.n_q):
        n_cb = O.visible_tokens(int(qp[0, i]), n_kv) // wl.c
        if n_cb:
            idx[0, i, :min(2, n_cb)] = rng.choice(n_cb, size=min(2, n_cb), replace=False)
    for name, sel in (("dense", None), ("blocks", idx)):
        got = dsa.sparse_attn(d["Q"], d["K"], d["V"], d["q_pos"],
                              None if sel is None else torch.from_numpy(sel.astype(np.int32)).to(DEV),
                              c=wl.c, scale=wl.scale).cpu().double().numpy()
        ref = O.sparse_attention(f64(x["Q"]), f64(x["K"]), f64(x["V"]), sel, qp, kv, wl.c, wl.scale)
        err = float(np.nanmax(np.abs(got - np.nan_to_num(ref))))
        print(f"gqa query tiles, {n_kv} keys, {name}: max |O - oracle| {err:.2e}")
        assert err <= 2e-2
