"""Parity of the indexer-key cache write (dsa_index_key_write, through the C
ABI) with the CPU oracle.

The stored rows are integers decided by float32 arithmetic whose every step
is fixed (fast Walsh-Hadamard butterflies in a set order, correctly rounded
f32 division, round-to-nearest-even codes), so the bar is bit-exact: every
f16 / bf16 / fp8 byte and every f32 row scale.  Rows the call must not touch
keep a sentinel pattern.
"""

import numpy as np
import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from oracle import dsa_oracle as O
from sparse_top_attention_indexer_amd import inputs
from test_parity_gpu import rel_err   # the suite's score tolerance rule

pytestmark = pytest.mark.gpu
DEV = "cuda"
CACHE = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
SENTINEL_SCALE = -7.0


def sentinel_cache(S, n_cache, name):
    if name == "fp8":
        c = torch.full((S, n_cache, 128), 0x5A, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
        sc = torch.full((S, n_cache), SENTINEL_SCALE, dtype=torch.float32, device=DEV)
        return c, sc
    c = torch.full((S, n_cache, 128), 0x5A5A, dtype=torch.int16, device=DEV).view(CACHE[name])
    return c, None


def bits(t):
    t = t.cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def expected(k_new, dst, n_cache, name, hadamard):
    """The oracle's rows placed at their destinations over the sentinel."""
    S, n_new, _ = k_new.shape
    rows, scale = O.index_key_write(O.to_f64(k_new).astype(np.float32), name, hadamard)
    if name == "fp8":
        cache = np.full((S, n_cache, 128), 0x5A, dtype=np.uint8)
        sc = np.full((S, n_cache), SENTINEL_SCALE, dtype=np.float32)
    else:
        cache = np.full((S, n_cache, 128), 0x5A5A, dtype=np.uint16)
        sc = None
    for s in range(S):
        for t in range(n_new):
            r = t if dst is None else int(dst[s, t])
            if 0 <= r < n_cache:
                cache[s, r] = rows[s, t]
                if sc is not None:
                    sc[s, r] = scale[s, t]
    return cache, sc


def check(k_new, dst, n_cache, name, hadamard):
    S = k_new.shape[0]
    cache, scale = sentinel_cache(S, n_cache, name)
    dsa.index_key_write(k_new.to(DEV), cache, dst_row=None if dst is None else dst.to(DEV),
                        cache_scale=scale, hadamard=hadamard)
    torch.cuda.synchronize()
    ref, ref_scale = expected(k_new, None if dst is None else dst.numpy(), n_cache, name, hadamard)
    got = bits(cache)
    bad = int((got != ref).any(axis=-1).sum())
    assert bad == 0, f"{bad} cache rows differ from the oracle"
    if ref_scale is not None:
        assert np.array_equal(scale.cpu().numpy().view(np.uint32), ref_scale.view(np.uint32))


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("name", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("k_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_key_write_bitwise(k_dtype, name, hadamard):
    # 37 new keys (two partial 16-row workgroups), scattered rows, one zero row,
    # x8 outlier rows, two destinations outside the cache per sequence
    b = inputs.key_write_batch(3, 37, 100, k_dtype, seed=2001, outlier_frac=0.1)
    check(b["k_new"], b["dst_row"], 100, name, hadamard)


@pytest.mark.parametrize("n_new", [0, 1, 50])
def test_key_write_contiguous_rows(n_new):
    # dst_row NULL: rows 0 .. n_new - 1 (a fresh fill; n_new = 1 is one decode step)
    b = inputs.key_write_batch(8, n_new, 64, torch.bfloat16, seed=2002 + n_new)
    check(b["k_new"], None, 64, "fp8", True)


def test_key_write_long_decode_cache_sampled():
    # the long-decode index cache: 8 sequences x 131072 rotated fp8 rows, written in one call
    S, n = 8, 131072
    b = inputs.key_write_batch(S, n, n, torch.bfloat16, seed=2005, zero_rows=1, skipped=0)
    cache, scale = sentinel_cache(S, n, "fp8")
    dsa.index_key_write(b["k_new"].to(DEV), cache, cache_scale=scale, hadamard=True)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, n - 1], g.integers(0, n, 512)]))
    k = b["k_new"][:, rows]
    ref, ref_scale = O.index_key_write(O.to_f64(k).astype(np.float32), "fp8", True)
    got = bits(cache[:, rows])
    assert np.array_equal(got, ref)
    assert np.array_equal(scale[:, rows].cpu().numpy().view(np.uint32), ref_scale.view(np.uint32))


def test_written_cache_scores_like_the_oracle():
    # the written cache is what the indexer reads: rotated fp8 keys + scales, queries rotated in-kernel
    S, n = 2, 700
    b = inputs.key_write_batch(S, n, n, torch.bfloat16, seed=2006, skipped=0)
    cache, scale = sentinel_cache(S, n, "fp8")
    dsa.index_key_write(b["k_new"].to(DEV), cache, cache_scale=scale, hadamard=True)
    qw = inputs.indexer_queries(S, 5, 64, seed=2007)
    q, w = qw["q_idx"], qw["w"]
    q_pos = torch.tensor([[699, 500, 31, 0, 350]] * S, dtype=torch.int32)
    got = dsa.index_scores(q.to(DEV), cache, w.to(DEV), q_pos.to(DEV), k_scale=scale,
                           hadamard_q=True).cpu().double().numpy()
    codes, sc = O.index_key_write(O.to_f64(b["k_new"]).astype(np.float32), "fp8", True)
    keys = O.decode_fp8_e4m3fn(codes)
    qf, wf = O.to_f64(q), O.to_f64(w)
    ref = O.index_scores(qf, keys, wf, q_pos.numpy(), k_scale=sc.astype(np.float64), rotate_q=True)
    cond = O.index_scores(qf, keys, np.abs(wf), q_pos.numpy(), k_scale=sc.astype(np.float64), rotate_q=True)
    err = rel_err(got, ref, cond)
    print(f"written fp8 cache: max relative score error {err:.2e}")
    assert err <= 2e-2


def test_key_write_fp8_encoder_midpoints():
    # unrotated f32 rows whose largest magnitude is 448: the multiplier 448 / m is
    # exactly 1, so every other element reaches the e4m3fn rounding unchanged --
    # every value of the format, every midpoint between neighbours (ties to the
    # even code) and the subnormal range, with both signs
    table = O.decode_fp8_e4m3fn(np.arange(127, dtype=np.uint8))
    mids = (table[:-1] + table[1:]) / 2
    vals = np.concatenate([table, mids, np.arange(40) * 2.0 ** -11]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 127
    n_rows = -(-len(vals) // per)
    k = np.zeros((1, n_rows, 128), dtype=np.float32)
    for r in range(n_rows):
        chunk = vals[r * per:(r + 1) * per]
        k[0, r, 0] = 448.0
        k[0, r, 1:1 + len(chunk)] = chunk
    check(torch.from_numpy(k), None, n_rows, "fp8", False)
