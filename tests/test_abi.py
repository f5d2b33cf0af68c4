"""Host-side checks of the C ABI: the library loads, exports every function
include/dsa.h declares, descriptor layouts agree with the binding, and every
argument check fails before anything is launched.

The error-path calls pass fake (never dereferenced) device addresses, so they
run only where no GPU is visible."""

import ctypes
import os
import re

import pytest
import torch

import sparse_top_attention_indexer_amd as dsa
from sparse_top_attention_indexer_amd import AttnDesc, ForwardDesc, IndexDesc, TopkDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="error-path calls use fake device addresses")

OK, NULL, SHAPE, DTYPE, PARAM, ALIGN, WORKSPACE, HIP, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = 0x10000   # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", src)))


def test_header_functions_are_exported_and_bound():
    L = dsa.lib()
    names = declared_functions()
    assert "dsa_forward" in names and "dsa_topk" in names and len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
        assert n in dsa.SYMBOLS, n


def test_descriptor_layouts_match():
    L = dsa.lib()
    for which, cls in enumerate((IndexDesc, TopkDesc, AttnDesc, ForwardDesc)):
        assert L.dsa_desc_size(which) == ctypes.sizeof(cls)
    assert L.dsa_desc_size(7) == 0
    assert L.dsa_version() >= 100
    for code in (OK, NULL, SHAPE, DTYPE, PARAM, ALIGN, WORKSPACE, HIP, UNSUP, 42):
        assert isinstance(L.dsa_strerror(code), bytes)


def _index(**kw):
    d = IndexDesc(FAKE, FAKE, None, FAKE, FAKE, None, 1, 1, 1, 4, 64, 128, 1000, 1, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(w=None), NULL), (dict(q_pos=None), NULL),
    (dict(S=0), SHAPE), (dict(n_q=0), SHAPE), (dict(H=0), SHAPE), (dict(H=129), SHAPE),
    (dict(D=100), SHAPE), (dict(D=512), SHAPE), (dict(n_units=0), SHAPE),
    (dict(c=0), PARAM), (dict(hadamard_q=2), PARAM), (dict(hadamard_q=1, D=64), SHAPE),
    (dict(q_dtype=3), DTYPE), (dict(k_dtype=7), DTYPE),
    (dict(k_dtype=3), NULL),                      # fp8 keys need a scale
    (dict(k_scale=FAKE), PARAM),                  # a scale without fp8 keys
    (dict(q=FAKE + 4), ALIGN), (dict(k=FAKE + 8), ALIGN),
])
def test_index_scores_rejects(kw, code):
    L = dsa.lib()
    assert L.dsa_index_scores(ctypes.byref(_index(**kw)), ctypes.c_void_p(FAKE), None) == code
    assert L.dsa_index_scores(None, ctypes.c_void_p(FAKE), None) == NULL
    assert L.dsa_index_scores(ctypes.byref(_index()), None, None) == NULL


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q_pos=None), NULL), (dict(S=0), SHAPE), (dict(n_units=0), SHAPE),
    (dict(top_k=0), PARAM), (dict(c=0), PARAM), (dict(c=3, top_k=64), PARAM),
    (dict(n_sink=-1), PARAM), (dict(n_sink=65), PARAM), (dict(c=4, n_sink=1), PARAM),
])
def test_topk_rejects(kw, code):
    L = dsa.lib()
    d = TopkDesc(FAKE, None, 1, 4, 1000, 64, 1, 0, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    assert L.dsa_topk(ctypes.c_void_p(FAKE), ctypes.byref(d), ctypes.c_void_p(FAKE), None, 0, None) == code


@no_gpu
@pytest.mark.parametrize("kw,code", [({"top_k": 0}, PARAM), ({"S": 0}, SHAPE), ({"q_pos": None}, NULL),
                                     ({"S": 17, "n_q": 1, "n_units": 131072, "top_k": 2048}, WORKSPACE)])
def test_topk_noalloc_rejects(kw, code):
    # the same argument checks as dsa_topk, and a workspace beyond the 16 MiB
    # static scratch is refused before the scratch is even looked up
    L = dsa.lib()
    d = TopkDesc(FAKE, None, 1, 4, 1000, 64, 1, 0, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    assert L.dsa_topk_noalloc(ctypes.c_void_p(FAKE), ctypes.byref(d), ctypes.c_void_p(FAKE), None) == code
    assert L.dsa_topk_noalloc(None, ctypes.byref(d), ctypes.c_void_p(FAKE), None) == NULL


@no_gpu
def test_topk_workspace_rule():
    L = dsa.lib()
    short = TopkDesc(FAKE, None, 1, 4096, 4096, 2048, 1, 0, 0)
    long = TopkDesc(FAKE, None, 8, 1, 131072, 2048, 1, 0, 0)
    assert L.dsa_topk_workspace_bytes(ctypes.byref(short)) == 0
    need = L.dsa_topk_workspace_bytes(ctypes.byref(long))
    assert need >= 8 * 131072 * 8
    assert L.dsa_topk(ctypes.c_void_p(FAKE), ctypes.byref(long), ctypes.c_void_p(FAKE), None, need,
                      None) == WORKSPACE
    assert L.dsa_topk(ctypes.c_void_p(FAKE), ctypes.byref(long), ctypes.c_void_p(FAKE),
                      ctypes.c_void_p(FAKE), need - 1, None) == WORKSPACE
    assert L.dsa_topk(ctypes.c_void_p(FAKE), ctypes.byref(long), ctypes.c_void_p(FAKE),
                      ctypes.c_void_p(FAKE + 8), need, None) == ALIGN   # the workspace is 16-byte aligned too


@no_gpu
def test_block_pool_rejects():
    L = dsa.lib()
    f = ctypes.c_void_p(FAKE)
    assert L.dsa_block_pool(None, 1, 1, 100, 128, 4, f, None) == NULL
    assert L.dsa_block_pool(f, 3, 1, 100, 128, 4, f, None) == DTYPE
    assert L.dsa_block_pool(f, 1, 0, 100, 128, 4, f, None) == SHAPE
    assert L.dsa_block_pool(f, 1, 1, 100, 128, 0, f, None) == PARAM


def _mla(**kw):
    d = AttnDesc(FAKE, FAKE, FAKE, 1000 * 576, 576, 576, 1000 * 576, 576, 576, FAKE, None,
                 1, 0, 1, 4, 128, 1, 576, 512, 1000, 64, 1, 0.0, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(q_pos=None), NULL), (dict(S=0), SHAPE), (dict(Hq=100), UNSUP),
    (dict(Hkv=3), SHAPE), (dict(n_kv=0), SHAPE), (dict(o_dtype=2), DTYPE), (dict(dtype=2), DTYPE),
    (dict(c=0), PARAM), (dict(k_sel=0), SHAPE), (dict(c=4, k_sel=5000), SHAPE),
    (dict(c=4, k_sel=1025), SHAPE),               # MLA keeps at most 1024 block ids per row
    (dict(n_kv=8 * 1024 * 1024), UNSUP),          # MLA row offsets within a sequence stay 32-bit
    (dict(v=FAKE + 1024), UNSUP),                 # MLA values must alias the latent rows
    (dict(Dk=64, Dv=64), UNSUP), (dict(k_tok_stride=-1), SHAPE),
    (dict(k_tok_stride=577, v_tok_stride=577), ALIGN), (dict(q=FAKE + 2), ALIGN),
])
def test_sparse_attn_rejects(kw, code):
    L = dsa.lib()
    d = _mla(**kw)
    assert L.dsa_sparse_attn(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, 0,
                             None) == code


@no_gpu
def test_sparse_attn_workspace_rule():
    L = dsa.lib()
    decode = _mla(S=8, n_q=1, n_kv=131072, k_sel=2048)
    need = L.dsa_sparse_attn_workspace_bytes(ctypes.byref(decode), 0)
    assert need > 0            # few rows: the stream is split and merged
    assert L.dsa_sparse_attn(ctypes.byref(decode), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), need - 4, None) == WORKSPACE
    assert L.dsa_sparse_attn(ctypes.byref(decode), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE + 4), need, None) == ALIGN
    prefill = _mla(S=1, n_q=4096, n_kv=4096, k_sel=2048)
    assert L.dsa_sparse_attn_workspace_bytes(ctypes.byref(prefill), 0) == 0


def _fwd(**kw):
    d = ForwardDesc(FAKE, FAKE, None, FAKE, 1, 1, 64, 128, 2048, 1, 0, 0,
                    FAKE, FAKE, FAKE, 4096 * 576, 576, 576, 4096 * 576, 576, 576,
                    1, 0, 128, 1, 576, 512, 0.0, 0, 1, 4096, 4096, FAKE, None, FAKE, None, None, None)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(w=None), NULL), (dict(top_k=0), PARAM),
    (dict(c=64, top_k=100), PARAM), (dict(c=64, n_sink=1), PARAM), (dict(n_sink=4096), PARAM),
    (dict(c=64, k_idx_dtype=3, k_scale=FAKE), DTYPE), (dict(k_idx_dtype=3), NULL),
    (dict(H=200), SHAPE), (dict(Hq=96, Dk=128, Dv=128, Hkv=1, v=FAKE), UNSUP),
    (dict(scores_out=FAKE + 4), ALIGN),
])
def test_forward_rejects(kw, code):
    L = dsa.lib()
    d = _fwd(**kw)
    assert L.dsa_forward(ctypes.byref(d), ctypes.c_void_p(FAKE), 1 << 40, None) == code


@no_gpu
def test_forward_workspace_covers_intermediates():
    L = dsa.lib()
    prefill = _fwd()
    need = L.dsa_forward_workspace_bytes(ctypes.byref(prefill))
    assert need >= 4096 * 4096 * 4 + 4096 * 2048 * 4   # scores + idx
    assert L.dsa_forward(ctypes.byref(prefill), ctypes.c_void_p(FAKE), need - 1, None) == WORKSPACE
    assert L.dsa_forward(ctypes.byref(prefill), None, need, None) == WORKSPACE
    assert L.dsa_forward(ctypes.byref(prefill), ctypes.c_void_p(FAKE + 8), need, None) == ALIGN


@no_gpu
def test_index_key_write_rejects():
    L = dsa.lib()
    f = ctypes.c_void_p(FAKE)

    def call(k=f, kd=1, S=2, n=10, D=128, dst=None, had=1, cache=f, cd=3, sc=f, nc=100):
        return L.dsa_index_key_write(k, kd, S, n, D, dst, had, cache, cd, sc, nc, None)

    assert call(k=None) == NULL and call(cache=None) == NULL
    assert call(cd=3, sc=None) == NULL                 # fp8 cache needs its scales
    assert call(cd=2, sc=f) == PARAM                   # scales without an fp8 cache
    assert call(kd=3) == DTYPE and call(cd=0, sc=None) == DTYPE and call(cd=9) == DTYPE
    assert call(S=0) == SHAPE and call(S=65536) == SHAPE and call(n=-1) == SHAPE and call(nc=0) == SHAPE and call(D=64) == SHAPE
    assert call(had=2) == PARAM
    assert call(k=ctypes.c_void_p(FAKE + 8)) == ALIGN and call(dst=ctypes.c_void_p(FAKE + 4)) == ALIGN
    assert call(n=0) == OK and call(k=None, n=0) == OK   # nothing to write: no launch


@no_gpu
def test_block_pool_update_rejects():
    L = dsa.lib()
    f = ctypes.c_void_p(FAKE)
    assert L.dsa_block_pool_update(f, 1, 1, 100, 128, 4, None, None, f, None) == NULL   # from_block is required
    assert L.dsa_block_pool_update(None, 1, 1, 100, 128, 4, f, None, f, None) == NULL
    assert L.dsa_block_pool_update(f, 3, 1, 100, 128, 4, f, None, f, None) == DTYPE
    assert L.dsa_block_pool_update(f, 1, 0, 100, 128, 4, f, None, f, None) == SHAPE
    assert L.dsa_block_pool_update(f, 1, 1, 100, 128, 0, f, None, f, None) == PARAM
    assert L.dsa_block_pool_update(ctypes.c_void_p(FAKE + 2), 1, 1, 100, 128, 4, f, None, f, None) == ALIGN
    assert L.dsa_block_pool(f, 1, 1, 100, 128, 4, ctypes.c_void_p(FAKE + 4), None) == ALIGN


def test_index_share_rule_matches_the_oracle():
    # host-only export: the layer rule, no launch
    from oracle import dsa_oracle as O
    L = dsa.lib()
    assert L.dsa_index_share_source(-1) == PARAM
    assert [L.dsa_index_share_source(il) for il in range(200)] == [O.index_share_source(il) for il in range(200)]


@no_gpu
def test_q8_latent_attention_rejects():
    # q8_0 latent rows: the MLA shapes only, with a Q of bf16 and the scales given
    L = dsa.lib()

    def attn(**kw):
        d = AttnDesc(FAKE, FAKE, FAKE, 576 * 100, 576, 576, 576 * 100, 576, 576, FAKE, None, 1, 0,
                     1, 1, 128, 1, 576, 512, 100, 64, 1, 0.0, 4, FAKE)
        for k, v in kw.items():
            setattr(d, k, v)
        return L.dsa_sparse_attn(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, 0, None)

    assert attn(kv_scale=None) == NULL
    assert attn(dtype=0) == DTYPE                 # Q must be bf16
    assert attn(kv_format=7) == DTYPE
    assert attn(Dk=128, Dv=128) == UNSUP          # q8_0 rows are MLA latents only
    assert attn(Hkv=2, Hq=128) == UNSUP
    assert attn(kv_scale=FAKE + 4) == ALIGN
    assert attn(k_tok_stride=584, v_tok_stride=584) == ALIGN   # byte rows on 16-byte boundaries
