"""Pins of the CPU oracle against things other than itself.

Brute force on tiny inputs, closed forms, library routines (numpy/torch on the
CPU) and invariants the pages fix.  Each test is chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, ReLU after instead of before the head sum, a wrong tie rule or head
grouping) fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoding --

def test_fp8_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_fp8_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed-form spot values of the e4m3fn encoding
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_16bit_decode_matches_torch_all_patterns(kind):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if kind == "bf16":
        ours = O.decode_bf16(bits)
        ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    else:
        ours = O.decode_f16(bits)
        ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ---------------------------------------------------------------- Hadamard --

def test_hadamard_closed_form_and_involution():
    n = 128
    H = O.hadamard(n)
    i = np.arange(n)
    pop = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    closed = np.where(pop % 2 == 0, 1.0, -1.0) / math.sqrt(n)
    assert np.array_equal(H, closed)                      # Sylvester entries
    assert np.allclose(H @ H, np.eye(n), atol=1e-14, rtol=0)   # H.H = I
    assert np.array_equal(H, H.T)
    with pytest.raises(ValueError):
        O.hadamard(96)


# ------------------------------------------------------------------ scores --

def _brute_scores(q, k, w, q_pos, kv_len, key_scale=None):
    """Scalar loops, written independently of the vectorised oracle."""
    S, n_q, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    n_k = len(k[0])
    out = [[[-math.inf] * n_k for _ in range(n_q)] for _ in range(S)]
    for s in range(S):
        for i in range(n_q):
            for j in range(n_k):
                if j > q_pos[s][i] or j >= kv_len[s]:
                    continue
                tot = 0.0
                for h in range(H):
                    dot = 0.0
                    for d in range(D):
                        kv = k[s][j][d] * (key_scale[s][j] if key_scale is not None else 1.0)
                        dot += q[s][i][h][d] * kv
                    if dot > 0.0:
                        tot += w[s][i][h] * dot
                out[s][i][j] = tot
    return np.array(out)


def test_scores_match_scalar_brute_force():
    rng = np.random.default_rng(0)
    S, n_q, H, D, n_k = 2, 5, 3, 8, 7
    q = rng.standard_normal((S, n_q, H, D))
    k = rng.standard_normal((S, n_k, D))
    w = rng.standard_normal((S, n_q, H))
    ks = rng.uniform(0.5, 2.0, (S, n_k))
    q_pos = np.array([[0, 2, 3, 6, 9], [-1, 1, 4, 5, 6]])
    kv_len = [7, 5]
    ours = O.index_scores(q, k, w, q_pos, kv_len, 1, ks)
    ref = _brute_scores(q.tolist(), k.tolist(), w.tolist(), q_pos.tolist(), kv_len, ks.tolist())
    assert np.array_equal(np.isinf(ours), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.allclose(ours[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_scores_relu_before_head_sum_golden():
    g = json.load(open(os.path.join(GOLDEN, "relu_before_head_sum.json")))
    s = O.index_scores(np.array(g["q"]), np.array(g["k"]), np.array(g["w"]),
                       np.array(g["q_pos"]))
    assert np.array_equal(s, np.array(g["expected_scores"]))
    idx = O.topk(s, np.array(g["q_pos"]), 1)
    assert idx.tolist() == g["expected_top1"]


def test_scores_single_head_reduce_to_relu_matmul():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 6, 1, 16))
    k = rng.standard_normal((1, 9, 16))
    s = O.index_scores(q, k, np.ones((1, 6, 1)), np.full((1, 6), 100))
    ref = torch.relu(torch.from_numpy(q[0, :, 0]) @ torch.from_numpy(k[0]).T).numpy()
    assert np.allclose(s[0], ref, rtol=1e-13, atol=1e-13)


def test_scores_invariant_under_hadamard_rotation():
    rng = np.random.default_rng(2)
    D = 128
    q = rng.standard_normal((2, 3, 4, D))
    k = rng.standard_normal((2, 50, D))
    w = rng.standard_normal((2, 3, 4))
    qp = np.array([[10, 30, 49], [0, 25, 60]])
    H = O.hadamard(D)
    plain = O.index_scores(q, k, w, qp)
    rotated = O.index_scores(q, k @ H.T, w, qp, rotate_q=True)
    fin = np.isfinite(plain)
    assert np.array_equal(fin, np.isfinite(rotated))
    assert np.allclose(plain[fin], rotated[fin], rtol=1e-12, atol=1e-10)
    # rotating only one side does change the scores
    one_side = O.index_scores(q, k @ H.T, w, qp)
    assert not np.allclose(plain[fin], one_side[fin], rtol=1e-3)


def test_scores_homogeneous_in_key_scale_and_linear_in_w():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((20, 32))
    w1, w2 = rng.standard_normal(4), rng.standard_normal(4)
    a = rng.uniform(0.1, 5.0, 20)
    base = O.index_scores_row(q, w1, k, 20)
    assert np.allclose(O.index_scores_row(q, w1, k, 20, key_scale=a), a * base, rtol=1e-12)
    s12 = O.index_scores_row(q, w1 + w2, k, 20)
    assert np.allclose(s12, base + O.index_scores_row(q, w2, k, 20), rtol=1e-11, atol=1e-11)
    # a negative key scale is not homogeneous: the ReLU sees the sign
    assert not np.allclose(O.index_scores_row(q, w1, -k, 20), -base)


def test_scores_visibility():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 3, 2, 8))
    k = rng.standard_normal((1, 10, 8))
    w = np.abs(rng.standard_normal((1, 3, 2))) + 0.1
    s = O.index_scores(q, k, w, np.array([[-1, 3, 20]]), kv_len=[6])
    assert np.all(np.isneginf(s[0, 0]))
    assert np.all(np.isfinite(s[0, 1, :4])) and np.all(np.isneginf(s[0, 1, 4:]))
    assert np.all(np.isfinite(s[0, 2, :6])) and np.all(np.isneginf(s[0, 2, 6:]))
    # block units: block b visible iff its last position is visible
    sb = O.index_scores(q, k[:, :5], w, np.array([[6, 7, 9]]), kv_len=[10], c=2)
    assert np.isfinite(sb[0, 0]).sum() == 3 and np.isfinite(sb[0, 1]).sum() == 4
    assert np.isfinite(sb[0, 2]).sum() == 5


# ------------------------------------------------------------------- top-k --

def test_topk_maximises_sum_by_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 12))
        sc = rng.standard_normal(n)
        sel = O.topk_row(sc, n, k)
        K = min(k, n)
        best = max(itertools.combinations(range(n), K), key=lambda c: sum(sc[list(c)]))
        assert sel.tolist() == sorted(best)


def test_topk_matches_torch_topk_on_distinct_scores():
    rng = np.random.default_rng(6)
    sc = rng.standard_normal(5000)
    sel = O.topk_row(sc, 4000, 777)
    ref = torch.topk(torch.from_numpy(sc[:4000]), 777).indices.sort().values.numpy()
    assert np.array_equal(sel, ref)


def test_topk_ties_go_to_lowest_index():
    assert O.topk_row(np.zeros(50), 50, 7).tolist() == list(range(7))
    sc = np.array([1.0, 5.0, 3.0, 5.0, 3.0, 3.0, 0.0])
    assert O.topk_row(sc, 7, 3).tolist() == [1, 2, 3]
    assert O.topk_row(sc, 7, 4).tolist() == [1, 2, 3, 4]


def test_topk_signed_zeros_are_equal_scores():
    # IEEE -0 == +0: zeros of either sign tie, and the tie goes to the lowest
    # index (a +0 after a -0 is not ranked above it)
    sc = np.array([-0.0, 0.0, -0.0, 0.0, 1.0, -0.0, -1.0])
    assert O.topk_row(sc, 7, 3).tolist() == [0, 1, 4]
    assert O.topk_row(sc, 7, 4).tolist() == [0, 1, 2, 4]
    assert O.topk_row(sc[::-1].copy(), 7, 3).tolist() == [1, 2, 3]


def test_topk_short_rows_keep_everything_and_pad():
    sc = np.array([[[0.3, -2.0, 1.0, 7.0, -np.inf, -np.inf]]])
    idx = O.topk(sc, np.array([[3]]), 5)
    assert idx.tolist() == [[[0, 1, 2, 3, -1]]]
    idx = O.topk(sc, np.array([[-1]]), 5)
    assert idx.tolist() == [[[-1] * 5]]


def test_topk_sink_is_forced():
    sc = np.array([-100.0, 5.0, 4.0, 3.0, 2.0, 1.0])
    assert O.topk_row(sc, 6, 3, n_sink=1).tolist() == [0, 1, 2]
    assert O.topk_row(sc, 6, 3, n_sink=2).tolist() == [0, 1, 2]
    sc2 = np.array([-100.0, -50.0, 4.0, 3.0, 2.0, 1.0])
    assert O.topk_row(sc2, 6, 3, n_sink=2).tolist() == [0, 1, 2]
    assert O.topk_row(sc2, 6, 3, n_sink=0).tolist() == [2, 3, 4]
    # the sink equals a +1e20 boost of the first keys when n_sink <= k
    boosted = sc2.copy()
    boosted[:2] += 1e20
    assert O.topk_row(boosted, 6, 3).tolist() == O.topk_row(sc2, 6, 3, n_sink=2).tolist()


def test_topk_rows_are_independent():
    rng = np.random.default_rng(7)
    sc = rng.standard_normal((3, 4, 40))
    qp = rng.integers(-1, 45, (3, 4))
    kv = [40, 33, 12]
    batched = O.topk(sc, qp, 9, kv, n_sink=1)
    for s in range(3):
        alone = O.topk(sc[s:s + 1], qp[s:s + 1], 9, [kv[s]], n_sink=1)
        assert np.array_equal(alone[0], batched[s])


# -------------------------------------------------------------- block mode --

def test_block_pool_against_numpy_mean_and_constants():
    rng = np.random.default_rng(8)
    kr = rng.standard_normal((2, 37, 16))
    p = O.block_pool(kr, 8)
    assert p.shape == (2, 4, 16)
    ref = kr[:, :32].reshape(2, 4, 8, 16).mean(axis=2)
    assert np.allclose(p, ref, rtol=1e-14, atol=1e-15)
    const = np.broadcast_to(np.arange(5.0)[None, :, None], (1, 5, 3)).repeat(4, axis=1)
    assert np.array_equal(O.block_pool(const, 4)[0, :, 0], np.arange(5.0))
    assert np.array_equal(O.block_pool(kr, 1), kr)


def _block_case(n_vis, top_k, c, seed=9, H=4, D=16):
    rng = np.random.default_rng(seed)
    n_kv = n_vis + 5
    q = rng.standard_normal((1, 1, H, D))
    kr = rng.standard_normal((1, n_kv, D))
    w = rng.standard_normal((1, 1, H))
    qp = np.array([[n_vis - 1]])
    pooled = O.block_pool(kr, c)
    s = O.index_scores(q, pooled, w, qp, kv_len=[n_kv], c=c)
    blocks = O.topk(s, qp, top_k // c, kv_len=[n_kv], c=c)
    toks = O.block_token_set(blocks[0, 0], c, n_vis - 1, n_kv)
    return s, blocks, toks


@pytest.mark.parametrize("c,top_k", [(4, 8), (16, 64), (64, 256)])
def test_block_mode_dense_threshold(c, top_k):
    # exactly dense below top_k + c - 1 cached tokens ...
    n = top_k + c - 1
    _, _, toks = _block_case(n, top_k, c)
    assert sorted(toks.tolist()) == list(range(n))
    # ... and the first sparse length drops a whole block
    n = top_k + c
    _, blocks, toks = _block_case(n, top_k, c)
    assert len(toks) == n - c
    assert (blocks[0, 0] >= 0).sum() == top_k // c


def test_block_mode_cuts_on_block_boundaries_and_matches_token_expansion():
    c, top_k = 8, 24
    for seed in range(10):
        n_vis = 93
        s, blocks, toks = _block_case(n_vis, top_k, c, seed=seed)
        n_cb = n_vis // c
        tail = set(range(n_cb * c, n_vis))
        chosen = set(int(b) for b in blocks[0, 0] if b >= 0)
        body = set(toks.tolist()) - tail
        assert body == {b * c + t for b in chosen for t in range(c)}
        # second, independent path: give every token its block's score, take the
        # token top-(B*c) (block members tie, the budget is a whole number of
        # blocks, so the cut lands on a block boundary)
        tok_scores = np.repeat(s[0, 0, :n_cb], c)
        tsel = O.topk_row(tok_scores, n_cb * c, top_k)
        assert set(tsel.tolist()) == body


def test_block_mode_c1_is_token_mode():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 3, 2, 8))
    k = rng.standard_normal((1, 20, 8))
    w = rng.standard_normal((1, 3, 2))
    qp = np.array([[5, 12, 19]])
    s1 = O.index_scores(q, O.block_pool(k, 1), w, qp, c=1)
    assert np.array_equal(s1, O.index_scores(q, k, w, qp))
    idx = O.topk(s1, qp, 4)
    for i in range(3):
        a = O.block_token_set(idx[0, i], 1, int(qp[0, i]), 20)
        b = O.token_list(idx[0, i], int(qp[0, i]), 20)
        assert np.array_equal(a, b)


# --------------------------------------------------------------- attention --

def _sdpa_ref(Q, K, V, q_pos, kv_len, scale):
    """torch scaled_dot_product_attention on the CPU in fp64, explicit mask."""
    S, n_q, Hq, Dk = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    out = np.zeros((S, n_q, Hq, V.shape[3]))
    for s in range(S):
        q = torch.from_numpy(Q[s]).permute(1, 0, 2)                    # [Hq, n_q, Dk]
        k = torch.from_numpy(K[s]).permute(1, 0, 2).repeat_interleave(G, 0)
        v = torch.from_numpy(V[s]).permute(1, 0, 2).repeat_interleave(G, 0)
        j = torch.arange(K.shape[1])
        mask = (j[None, :] <= torch.from_numpy(q_pos[s])[:, None]) & (j[None, :] < kv_len[s])
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                             scale=scale)
        out[s] = o.permute(1, 0, 2).numpy()
    return out


def test_dense_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(11)
    S, n_q, n_kv, Hq, Hkv, D = 2, 6, 15, 8, 2, 16
    Q = rng.standard_normal((S, n_q, Hq, D))
    K = rng.standard_normal((S, n_kv, Hkv, D))
    V = rng.standard_normal((S, n_kv, Hkv, 12))
    qp = np.array([[0, 3, 7, 9, 14, 20], [2, 2, 5, 8, 11, 13]])
    kv = [15, 10]
    ours = O.dense_attention(Q, K, V, qp, kv, scale=0.3)
    ref = _sdpa_ref(Q, K, V, qp, kv, 0.3)
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_mla_values_alias_latent_rows():
    rng = np.random.default_rng(12)
    lat = rng.standard_normal((1, 30, 1, 40))
    Q = rng.standard_normal((1, 3, 4, 40))
    qp = np.array([[5, 17, 29]])
    ours = O.dense_attention(Q, lat, lat[..., :32], qp)
    ref = _sdpa_ref(Q, lat, np.ascontiguousarray(lat[..., :32]), qp, [30], 1 / math.sqrt(40))
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_exactly_when_topk_covers_everything():
    rng = np.random.default_rng(13)
    S, n_q, n_kv = 1, 20, 20
    Q = rng.standard_normal((S, n_q, 4, 16))
    K = rng.standard_normal((S, n_kv, 2, 16))
    V = rng.standard_normal((S, n_kv, 2, 16))
    q_idx = rng.standard_normal((S, n_q, 3, 32))
    k_idx = rng.standard_normal((S, n_kv, 32))
    w = rng.standard_normal((S, n_q, 3))
    qp = np.arange(n_q)[None, :]
    o_sparse, idx, _ = O.forward(Q, K, V, q_idx, k_idx, w, 32, 1, qp)
    o_dense = O.dense_attention(Q, K, V, qp)
    assert np.array_equal(o_sparse, o_dense)
    # block mode below the threshold (top_k + c - 1 = 23 >= 20 tokens) is dense too
    o_blk, _, _ = O.forward(Q, K, V, q_idx, k_idx, w, 20, 4, qp)
    assert np.array_equal(o_blk, o_dense)


def test_single_selected_key_returns_its_value():
    rng = np.random.default_rng(14)
    Q = rng.standard_normal((1, 1, 4, 8))
    K = rng.standard_normal((1, 10, 1, 8))
    V = rng.standard_normal((1, 10, 1, 8))
    o = O.sparse_attention(Q, K, V, np.array([[[6]]]), np.array([[9]]))
    assert np.array_equal(o[0, 0], np.repeat(V[0, 6], 4, axis=0))
    # empty and invisible selections give zero rows, never NaN
    o = O.sparse_attention(Q, K, V, np.array([[[-1]]]), np.array([[9]]))
    assert np.array_equal(o, np.zeros_like(o))
    o = O.sparse_attention(Q, K, V, np.array([[[3]]]), np.array([[-1]]))
    assert np.array_equal(o, np.zeros_like(o))


def test_attention_token_order_only_changes_rounding():
    rng = np.random.default_rng(15)
    Q = rng.standard_normal((1, 1, 4, 8))
    K = rng.standard_normal((1, 40, 2, 8))
    V = rng.standard_normal((1, 40, 2, 8))
    a = O.sparse_attention(Q, K, V, np.array([[[3, 9, 17, 30, 31]]]), np.array([[39]]))
    b = O.sparse_attention(Q, K, V, np.array([[[31, 17, 3, 30, 9]]]), np.array([[39]]))
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------ indexer-key cache write --

def test_rounding_to_16_bit_formats_is_single_and_to_even():
    # f16: numpy's float64 -> float16 conversion is one correct rounding; bf16:
    # torch's float32 -> bfloat16 cast is one on float32 inputs
    g = np.random.default_rng(11)
    v = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-6, 4, 20000),
                        [0.0, -0.0, 2.0 ** -24, 2.0 ** -25 * 3, 65504.0, -1.0]])
    assert np.array_equal(O.encode_f16_bits(v), v.astype(np.float16).view(np.uint16))
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.encode_bf16_bits(v32.astype(np.float64)), ref)
    # a value just above a bf16 midpoint by less than float32 resolution
    # rounds up (rounding through float32 first would tie and go to the even 1.0)
    assert O.decode_bf16(O.encode_bf16_bits(np.array([1 + 2.0 ** -8 + 2.0 ** -40])))[0] == 1 + 2.0 ** -7
    # exact midpoints tie to the even neighbour
    assert O.decode_bf16(O.encode_bf16_bits(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))).tolist() == [1.0, 1 + 2 * 2.0 ** -7]
    # 1/sqrt(128) = 1.41421356... * 2^-4: the 8-bit significand 181/128 (bf16
    # 0x3DB5), the 11-bit significand 1448/1024 (f16 0x2DA8), worked by hand
    c = np.array([1 / math.sqrt(128)])
    assert O.encode_bf16_bits(c)[0] == 0x3DB5 and O.encode_f16_bits(c)[0] == 0x2DA8


def test_key_write_16bit_of_basis_vectors():
    # H e_j is column j of H: entries +-1/sqrt(128), so every stored element is
    # +-0x3DB5 (bf16) or +-0x2DA8 (f16) with the sign pattern of the Sylvester matrix
    eye = np.eye(128)
    sign = O.hadamard(128) * math.sqrt(128)
    for name, mag in (("bf16", 0x3DB5), ("f16", 0x2DA8)):
        bits, none = O.index_key_write(eye, name, True)
        assert none is None
        want = np.where(sign.T > 0, mag, mag | 0x8000)
        assert np.array_equal(bits, want.astype(np.uint16))
        plain, _ = O.index_key_write(eye, name, False)   # unrotated: 1.0 and 0.0
        one = 0x3F80 if name == "bf16" else 0x3C00
        assert np.array_equal(plain, (np.eye(128) * one).astype(np.uint16))


def test_key_write_rotation_is_the_sylvester_product():
    # rotating twice gives the keys back (H.H = I), and a rotated query scores the
    # stored rotated keys like the plain ones (to the storage precision)
    g = np.random.default_rng(12)
    k = g.standard_normal((16, 128))
    assert np.abs(O.rotate_keys(O.rotate_keys(k, True), True) - k).max() < 1e-12
    assert np.array_equal(O.rotate_keys(k, False), k)
    bits16, _ = O.index_key_write(k, "f16", True)
    q = g.standard_normal((3, 128))
    d_rot = (q @ O.hadamard(128)) @ O.decode_f16(bits16).T
    assert np.abs(d_rot - q @ k.T).max() < 2e-2


def test_fp8_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn cast (round to nearest even) for finite in-range values,
    # including every exact midpoint between neighbouring codes and the subnormal range
    g = np.random.default_rng(13)
    vals = [g.uniform(-448, 448, 20000), g.standard_normal(20000) * 1e-2, g.uniform(-2**-6, 2**-6, 5000)]
    table = O.decode_fp8_e4m3fn(np.arange(127, dtype=np.uint8))
    mids = (table[:-1] + table[1:]) / 2
    vals += [mids, -mids, table, -table, [0.0, -0.0]]
    v = np.concatenate([np.asarray(a, dtype=np.float64) for a in vals]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_fp8_e4m3fn(v), ref)


def test_fp8_encode_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.encode_fp8_e4m3fn(O.decode_fp8_e4m3fn(codes).astype(np.float32)), codes)
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e6, -500.0], dtype=np.float32)
    assert list(O.encode_fp8_e4m3fn(big)) == [0x7E] * 5 + [0xFE]
    # ties go to the even code: 0.5 * (1 + 1.125) lies halfway between codes 0x38 and 0x39
    assert O.encode_fp8_e4m3fn(np.float32(1.0625))[()] == 0x38
    assert O.encode_fp8_e4m3fn(np.float32(1.1875))[()] == 0x3A   # between 0x39 and 0x3A: even wins


def test_key_write_fp8_closed_forms():
    # x = e_0: H x = 1/sqrt(128) in every element, so scale = (1/sqrt(128)) / 448
    # and every code is 448 (0x7E); x = e_0 - e_1: H x is 0 on even and
    # 2/sqrt(128) on odd elements (Sylvester order), so codes 0 and 448
    k = np.zeros((3, 128))
    k[0, 0] = 1.0
    k[1, 0], k[1, 1] = 1.0, -1.0
    codes, scale = O.index_key_write(k, "fp8", True)
    assert scale[0] == (1 / math.sqrt(128)) / 448 and np.all(codes[0] == 0x7E)
    assert scale[1] == (2 / math.sqrt(128)) / 448
    assert np.all(codes[1, 0::2] == 0) and np.all(codes[1, 1::2] == 0x7E)
    assert scale[2] == 0 and not codes[2].any()       # a zero row: scale 0, zero codes
    # unrotated: the scale is the row's max / 448 and that element stores +-448
    k2 = np.array([[3.0, -6.0] + [0.5] * 126])
    c2, s2 = O.index_key_write(k2, "fp8", False)
    assert s2[0] == 6.0 / 448 and c2[0, 1] == 0xFE and c2[0, 0] == O.encode_fp8_e4m3fn(np.array([224.0]))[0]


def test_key_write_fp8_bounds_and_extremes():
    g = np.random.default_rng(14)
    k = g.standard_normal((40, 128)).astype(np.float32).astype(np.float64)
    k[3] *= 8.0
    k[5] = 0.0
    for rot in (False, True):
        codes, scale = O.index_key_write(k, "fp8", rot)
        y = k @ O.hadamard(128).T if rot else k
        assert codes.dtype == np.uint8 and scale[5] == 0 and not codes[5].any()
        live = np.arange(40) != 5
        assert np.allclose(scale[live], np.abs(y[live]).max(-1) / 448, rtol=1e-15, atol=0)
        # the largest magnitude of each row is stored as +-448
        arg = np.abs(y[live]).argmax(-1)
        assert np.all((codes[live][np.arange(39), arg] & 0x7F) == 0x7E)
        # half a step of 3 mantissa bits (2^-10 absolute in the subnormal range), in scale units
        dec = O.decode_fp8_e4m3fn(codes) * scale[:, None]
        q = y / np.where(scale > 0, scale, 1)[:, None]
        bound = np.maximum(2.0 ** -4 * np.abs(q), 2.0 ** -10) * scale[:, None] * (1 + 1e-12)
        assert np.all(np.abs(dec - y) <= bound)


def test_key_write_check_accepts_the_oracle_and_rejects_plants():
    g = np.random.default_rng(15)
    k = g.standard_normal((24, 128)).astype(np.float32).astype(np.float64)
    k[2] *= 8.0
    k[4] = 0.0
    for name in ("f16", "bf16", "fp8"):
        for rot in (False, True):
            got, sc = O.index_key_write(k, name, rot)
            ok, exc = O.key_write_check(k, name, rot, got, None if sc is None else sc.astype(np.float32))
            assert ok.all() and exc == 0
            # one step off, on an element far from a rounding midpoint: rejected
            bad = got.copy()
            bad[7, 9] = bad[7, 9] + 1   # the next code / bit pattern up in magnitude
            ok2, _ = O.key_write_check(k, name, rot, bad, None if sc is None else sc.astype(np.float32))
            assert not ok2[7, 9] and ok2.sum() == ok2.size - 1
    # a scale off by more than the rounding bound marks its row
    got, sc = O.index_key_write(k, "fp8", True)
    sc2 = sc.astype(np.float32).copy()
    sc2[1] *= np.float32(1 + 2.0 ** -10)
    ok3, _ = O.key_write_check(k, "fp8", True, got, sc2)
    assert not ok3[1].any() and ok3[0].all()


def test_key_write_check_allows_the_other_neighbour_only_at_a_midpoint():
    # unrotated rows whose max is 448 put the values straight on the e4m3 grid:
    # an element at the exact midpoint 1.0625 of codes 0x38 (1.0) and 0x39
    # (1.125) rounds to the even 0x38, and 0x39 is valid too (a float32 path may
    # land on either side); at 1.04, far from any midpoint, only 0x38 is
    k = np.zeros((1, 128))
    k[0, 0], k[0, 1], k[0, 2] = 448.0, 1.0625, 1.04
    codes, sc = O.index_key_write(k, "fp8", False)
    assert codes[0, 1] == 0x38 and codes[0, 2] == 0x38
    alt = codes.copy()
    alt[0, 1] = 0x39
    ok, exc = O.key_write_check(k, "fp8", False, alt, sc.astype(np.float32))
    assert ok.all() and exc == 1
    alt[0, 2] = 0x39
    ok, _ = O.key_write_check(k, "fp8", False, alt, sc.astype(np.float32))
    assert not ok[0, 2]
    # the same for a bf16 row: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7
    k16 = np.array([[1 + 2.0 ** -8, 1 + 2.0 ** -9] + [0.0] * 126])
    bits, _ = O.index_key_write(k16, "bf16", False)
    assert bits[0, 0] == 0x3F80 and bits[0, 1] == 0x3F80
    b2 = bits.copy()
    b2[0, 0] = 0x3F81
    ok, exc = O.key_write_check(k16, "bf16", False, b2)
    assert ok.all() and exc == 1
    b2[0, 1] = 0x3F81
    ok, _ = O.key_write_check(k16, "bf16", False, b2)
    assert not ok[0, 1]


# ------------------------------------------------------ incremental block pooling --

def test_block_pool_update_equals_one_shot_after_micro_batches_and_an_edit():
    # micro-batches pool only what they complete; the result equals a one-shot
    # pool of the final keys, and blocks no update reached keep their value
    g = np.random.default_rng(31)
    S, n, D, c = 2, 100, 8, 8
    k = g.standard_normal((S, n, D))
    sentinel = np.full((S, n // c, D), -7.0)
    p = O.block_pool_update(k, c, sentinel, [0, 0], kv_len=[30, 0])
    assert np.allclose(p[0, :3], O.block_pool(k[:, :24], c)[0])   # 30 stored keys: 3 complete blocks
    assert np.all(p[0, 3:] == -7.0) and np.all(p[1] == -7.0)
    p = O.block_pool_update(k, c, p, [3, 0], kv_len=[100, 57])
    full = O.block_pool(k, c)
    assert np.allclose(p[0], full[0], rtol=0, atol=1e-15)
    assert np.allclose(p[1, :7], full[1, :7]) and np.all(p[1, 7:] == -7.0)
    # an edit of sequence 0 from position 41 stales its pools from block 5 on
    k2 = k.copy()
    k2[0, 41:] += 1.0
    p2 = O.block_pool_update(k2, c, p, [41 // c, 99], kv_len=[100, 57])
    assert np.array_equal(p2[0, :5], p[0, :5]) and np.allclose(p2[0, 5:], O.block_pool(k2, c)[0, 5:])
    assert np.array_equal(p2[1], p[1])
    # a constant block pools to its constant; a negative first block counts as 0
    kc = np.full((1, 16, 4), 2.5)
    assert np.all(O.block_pool_update(kc, 8, np.zeros((1, 2, 4)), [-3]) == 2.5)


# ------------------------------------------------------------- q8_0 latent --

def test_q8_0_decode_hand_worked_block():
    # one block with scale 0.5 (f16 0x3800) and codes -127, -1, 0, 1, 2, 127,
    # then 26 zeros; a second block with scale 2^-10 (f16 0x1400): codes x 2^-10
    codes = np.zeros(64, dtype=np.int8)
    codes[:6] = [-127, -1, 0, 1, 2, 127]
    codes[32:35] = [3, -64, 100]
    scales = np.array([0x3800, 0x1400], dtype=np.uint16)
    v = O.decode_q8_0(codes, scales)
    assert v[:6].tolist() == [-63.5, -0.5, 0.0, 0.5, 1.0, 63.5] and not v[6:32].any()
    assert v[32:35].tolist() == [3 / 1024, -64 / 1024, 100 / 1024] and not v[35:].any()
    # the same through f16 values instead of bit patterns
    assert np.array_equal(O.decode_q8_0(codes, scales.view(np.float16)), v)


def test_q8_0_encode_round_trip_bound_and_extremes():
    g = np.random.default_rng(41)
    x = g.standard_normal((50, 576))
    x[3] *= 8.0                          # an outlier row
    x[5, :32] = 0.0                      # a zero block
    x[7, 64:96] = np.linspace(-3, 3, 32)
    codes, scales = O.encode_q8_0(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float16 and scales.shape == (50, 18)
    assert scales[5, 0] == 0 and not codes[5, :32].any()
    dec = O.decode_q8_0(codes, scales)
    s = np.repeat(scales.astype(np.float64), 32, axis=-1)
    amax = np.repeat(np.abs(x.reshape(50, 18, 32)).max(-1), 32, axis=-1)
    # half a step, plus what the clamp at 127 can cut when the f16 scale
    # rounded below max / 127 (at most 127 s 2^-11)
    assert np.all(np.abs(dec - x) <= s / 2 + np.maximum(amax - 127 * s, 0) + 1e-12)
    # the largest element of every nonzero block reaches code +-127 or +-126 (f16 rounding of the scale)
    big = np.abs(codes.reshape(50, 18, 32)).max(-1)
    assert np.all((big >= 126) | (scales == 0))
    # halves round away from zero: 0.5 and -1.5 steps with scale 1
    xh = np.zeros(32)
    xh[0], xh[1], xh[2] = 127.0, 0.5, -1.5
    ch, sh = O.encode_q8_0(xh)
    assert sh[0] == 1.0 and ch[:3].tolist() == [127, 1, -2]


# ------------------------------------------------------------------ IndexShare --

def test_index_share_rule_reproduces_the_page_counts():
    # the IndexShare commit: the rule gives 21 full and 57 shared layers for the 78-layer model
    full = [il for il in range(78) if O.index_share_full(il)]
    assert len(full) == 21 and 78 - len(full) == 57
    assert full[:4] == [0, 1, 2, 6] and full[-1] == 74


def test_index_share_source_is_the_latest_full_layer():
    for il in range(78):
        src = O.index_share_source(il)
        assert O.index_share_full(src) and src <= il
        assert all(not O.index_share_full(j) for j in range(src + 1, il + 1))
    assert [O.index_share_source(il) for il in range(8)] == [0, 1, 2, 2, 2, 2, 6, 6]


def test_forward_layers_shares_selections():
    # shared layers attend over their source layer's rows: a stack whose layers
    # share one indexer input still gives each layer its own attention output
    g = np.random.default_rng(21)
    n, H, D, Hq, Dk = 40, 2, 128, 2, 16
    q_pos = np.arange(n)[None, :]
    layers = []
    for il in range(4):
        layers.append({"Q": g.standard_normal((1, n, Hq, Dk)), "K": g.standard_normal((1, n, Hq, Dk)),
                       "V": g.standard_normal((1, n, Hq, Dk)), "q_idx": g.standard_normal((1, n, H, D)),
                       "k_idx": g.standard_normal((1, n, D)), "w": g.random((1, n, H))})
    outs, idxs = O.forward_layers(layers, 8, 1, q_pos)
    assert np.array_equal(idxs[3], idxs[2])          # layer 3 is shared, its source is layer 2
    assert not np.array_equal(idxs[1], idxs[0])       # full layers select on their own
    want3 = O.sparse_attention(layers[3]["Q"], layers[3]["K"], layers[3]["V"], idxs[2], q_pos)
    assert np.array_equal(outs[3], want3)
    own3 = O.forward(*(layers[3][k] for k in ("Q", "K", "V", "q_idx", "k_idx", "w")), 8, 1, q_pos)[1]
    assert not np.array_equal(own3, idxs[3])          # ... which differs from what it would select itself
