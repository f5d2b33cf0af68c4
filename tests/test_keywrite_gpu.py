"""Parity of the indexer-key cache write (dsa_index_key_write, through the C
ABI) with the CPU oracle.

The oracle stores the exact rotated key rounded once into the cache type
(fp8: scale = max |H x| / 448, code = e4m3fn(H x / scale)).  The kernel
rotates in float32, as the pages do, so where an exact value lies within its
float32 rounding error of a midpoint of the cache type, it may take the other
neighbour: oracle.key_write_check states that rule, and every stored element
and every scale must pass it (the number of other-neighbour elements is
printed).  Rows the call must not touch keep a sentinel pattern.
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


def check_rows(x, got, got_scale, name, hadamard, what):
    """Every stored row valid under the oracle's rule; prints the exceptions."""
    ok, exc = O.key_write_check(x, name, hadamard, got, got_scale)
    bad = int((~ok).sum())
    print(f"{what}: {ok.size} elements, {exc} on the other neighbour of a midpoint, {bad} invalid")
    assert bad == 0, f"{bad} stored elements are not valid roundings of the rotated keys"
    return exc


def check(k_new, dst, n_cache, name, hadamard):
    S, n_new, _ = k_new.shape
    cache, scale = sentinel_cache(S, n_cache, name)
    dsa.index_key_write(k_new.to(DEV), cache, dst_row=None if dst is None else dst.to(DEV),
                        cache_scale=scale, hadamard=hadamard)
    torch.cuda.synchronize()
    got = bits(cache)
    got_scale = None if scale is None else scale.cpu().numpy()
    x = O.to_f64(k_new)
    written = np.zeros((S, n_cache), dtype=bool)
    xs, gs, ss = [], [], []
    for s in range(S):
        for t in range(n_new):
            r = t if dst is None else int(dst[s, t])
            if 0 <= r < n_cache:
                written[s, r] = True
                xs.append(x[s, t])
                gs.append(got[s, r])
                if got_scale is not None:
                    ss.append(got_scale[s, r])
    if xs:
        check_rows(np.stack(xs), np.stack(gs), np.array(ss) if ss else None, name, hadamard,
                   f"{name} rotate={hadamard} from {k_new.dtype}")
    sentinel = 0x5A if name == "fp8" else 0x5A5A
    assert np.all(got[~written] == sentinel), "a row outside the destinations was written"
    if got_scale is not None:
        assert np.all(got_scale[~written] == SENTINEL_SCALE)


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
    x = O.to_f64(b["k_new"][:, rows])
    check_rows(x, bits(cache[:, rows]), scale[:, rows].cpu().numpy(), "fp8", True, "long-decode cache rows")


def test_written_cache_scores_like_the_oracle():
    # the written cache is what the indexer reads: rotated fp8 keys + scales,
    # queries rotated in-kernel; the oracle scores the same stored codes and
    # scales (decoded exactly), after the rows pass the write rule
    S, n = 2, 700
    b = inputs.key_write_batch(S, n, n, torch.bfloat16, seed=2006, skipped=0)
    cache, scale = sentinel_cache(S, n, "fp8")
    dsa.index_key_write(b["k_new"].to(DEV), cache, cache_scale=scale, hadamard=True)
    torch.cuda.synchronize()
    codes, sc = bits(cache), scale.cpu().numpy()
    check_rows(O.to_f64(b["k_new"]).reshape(-1, 128), codes.reshape(-1, 128), sc.reshape(-1), "fp8", True,
               "written cache")
    qw = inputs.indexer_queries(S, 5, 64, seed=2007)
    q, w = qw["q_idx"], qw["w"]
    q_pos = torch.tensor([[699, 500, 31, 0, 350]] * S, dtype=torch.int32)
    got = dsa.index_scores(q.to(DEV), cache, w.to(DEV), q_pos.to(DEV), k_scale=scale,
                           hadamard_q=True).cpu().double().numpy()
    keys = O.decode_fp8_e4m3fn(codes)
    qf, wf = O.to_f64(q), O.to_f64(w)
    ref = O.index_scores(qf, keys, wf, q_pos.numpy(), k_scale=sc.astype(np.float64), rotate_q=True)
    # the condition scale sum_h |w_h| sum_d |q'_hd k_ud|, q' the rotated query
    qr = qf @ O.hadamard(128).T
    cond = O.index_scores(np.abs(qr), np.abs(keys), np.abs(wf), q_pos.numpy(), k_scale=sc.astype(np.float64))
    err = rel_err(got, ref, cond)
    print(f"written fp8 cache: max relative score error {err:.2e}")
    assert err <= 2e-2


def test_key_write_fp8_encoder_midpoints():
    # unrotated f32 rows whose largest magnitude is 448: the multiplier 448 / m is
    # exactly 1, so every other element reaches the e4m3fn rounding unchanged --
    # every value of the format, every midpoint between neighbours (ties to the
    # even code) and the subnormal range, with both signs.  No float32 error
    # enters, so the codes must be the oracle's exactly; the scales pass the rule
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
    cache, scale = sentinel_cache(1, n_rows, "fp8")
    dsa.index_key_write(torch.from_numpy(k).to(DEV), cache, cache_scale=scale, hadamard=False)
    torch.cuda.synchronize()
    want, _ = O.index_key_write(k.astype(np.float64), "fp8", False)
    got = bits(cache)
    # +0 and -0 codes are the same value
    same = (got == want) | (((got & 0x7F) == 0) & ((want & 0x7F) == 0))
    assert same.all(), f"{int((~same).sum())} codes differ from round-to-nearest-even"
    check_rows(k[0].astype(np.float64), got[0], scale.cpu().numpy()[0], "fp8", False, "encoder midpoints")
