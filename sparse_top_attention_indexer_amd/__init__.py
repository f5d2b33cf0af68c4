"""Python binding of the MI355X DSA library (libdsa.so).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors must live on the GPU; PyTorch provides device memory and the
current stream.  If the library is not built, every call raises.

Functions mirror the C entry points of include/dsa.h:
    index_scores, topk, block_pool, sparse_attn, forward
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

__all__ = ["index_scores", "topk", "topk_noalloc", "block_pool", "sparse_attn", "forward", "lib", "DsaError",
           "forward_workspace_bytes", "Event"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.float8_e4m3fn: 3}
Q8_0 = 4   # q8_0 latent rows: int8 codes + f16 scales per 32 values


class DsaError(RuntimeError):
    pass


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class IndexDesc(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("k_scale", _vp), ("w", _vp), ("q_pos", _vp), ("kv_len", _vp),
                ("q_dtype", _i32), ("k_dtype", _i32), ("S", _i32), ("n_q", _i32), ("H", _i32),
                ("D", _i32), ("n_units", _i64), ("c", _i32), ("hadamard_q", _i32)]


class TopkDesc(ctypes.Structure):
    _fields_ = [("q_pos", _vp), ("kv_len", _vp), ("S", _i32), ("n_q", _i32), ("n_units", _i64),
                ("top_k", _i32), ("c", _i32), ("n_sink", _i32), ("pad_", _i32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp),
                ("k_seq_stride", _i64), ("k_tok_stride", _i64), ("k_head_stride", _i64),
                ("v_seq_stride", _i64), ("v_tok_stride", _i64), ("v_head_stride", _i64),
                ("q_pos", _vp), ("kv_len", _vp), ("dtype", _i32), ("o_dtype", _i32),
                ("S", _i32), ("n_q", _i32), ("Hq", _i32), ("Hkv", _i32), ("Dk", _i32), ("Dv", _i32),
                ("n_kv", _i64), ("k_sel", _i32), ("c", _i32), ("scale", ctypes.c_float), ("kv_format", _i32),
                ("kv_scale", _vp)]


class ForwardDesc(ctypes.Structure):
    _fields_ = [("q_idx", _vp), ("k_idx", _vp), ("k_scale", _vp), ("w", _vp),
                ("q_idx_dtype", _i32), ("k_idx_dtype", _i32), ("H", _i32), ("D", _i32),
                ("top_k", _i32), ("c", _i32), ("n_sink", _i32), ("hadamard_q", _i32),
                ("q", _vp), ("k", _vp), ("v", _vp),
                ("k_seq_stride", _i64), ("k_tok_stride", _i64), ("k_head_stride", _i64),
                ("v_seq_stride", _i64), ("v_tok_stride", _i64), ("v_head_stride", _i64),
                ("a_dtype", _i32), ("o_dtype", _i32), ("Hq", _i32), ("Hkv", _i32), ("Dk", _i32),
                ("Dv", _i32), ("scale", ctypes.c_float), ("kv_format", _i32),
                ("S", _i32), ("n_q", _i32), ("n_kv", _i64), ("q_pos", _vp), ("kv_len", _vp),
                ("out", _vp), ("idx_out", _vp), ("scores_out", _vp), ("phase_events", _vp), ("kv_scale", _vp)]


SYMBOLS = {
    "dsa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "dsa_version": (ctypes.c_int, []),
    "dsa_desc_size": (ctypes.c_size_t, [ctypes.c_int]),
    "dsa_index_scores": (ctypes.c_int, [ctypes.POINTER(IndexDesc), _vp, _vp]),
    "dsa_topk_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(TopkDesc)]),
    "dsa_topk": (ctypes.c_int, [_vp, ctypes.POINTER(TopkDesc), _vp, _vp, ctypes.c_size_t, _vp]),
    "dsa_topk_noalloc": (ctypes.c_int, [_vp, ctypes.POINTER(TopkDesc), _vp, _vp]),
    "dsa_block_pool": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i32, _i32, _vp, _vp]),
    "dsa_block_pool_update": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "dsa_index_share_source": (ctypes.c_int32, [ctypes.c_int32]),
    "dsa_index_key_write": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i32, _vp, _i32, _vp, _i32, _vp, _i64, _vp]),
    "dsa_sparse_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AttnDesc), ctypes.c_int]),
    "dsa_sparse_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "dsa_forward_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ForwardDesc)]),
    "dsa_forward": (ctypes.c_int, [ctypes.POINTER(ForwardDesc), _vp, ctypes.c_size_t, _vp]),
    "dsa_event_create": (ctypes.c_int, [ctypes.POINTER(_vp)]),
    "dsa_event_destroy": (ctypes.c_int, [_vp]),
    "dsa_event_record": (ctypes.c_int, [_vp, _vp]),
    "dsa_event_elapsed_ms": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(ctypes.c_float)]),
}

_LIB = None


def lib():
    """The loaded libdsa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise DsaError(f"{LIB_PATH} is missing: build it with "
                           "sparse_top_attention_indexer_amd.build.build() (there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        for which, cls in enumerate((IndexDesc, TopkDesc, AttnDesc, ForwardDesc)):
            if L.dsa_desc_size(which) != ctypes.sizeof(cls):
                raise DsaError(f"descriptor {cls.__name__} layout mismatch with libdsa.so")
        _LIB = L
    return _LIB


def _check(status: int):
    if status != 0:
        raise DsaError(f"dsa error {status}: {lib().dsa_strerror(status).decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in DTYPES:
        raise DsaError(f"unsupported dtype {t.dtype}")
    return DTYPES[t.dtype]


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise DsaError("tensors must be on the GPU")


def _i32c(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise DsaError("positions and lengths must be contiguous int32 tensors")
    return t


# ------------------------------------------------------------------ scores --

def index_scores(q, k, w, q_pos, *, c: int = 1, k_scale=None, kv_len=None, hadamard_q: bool = False,
                 out=None):
    """Indexer scores [S, n_q, n_units] f32 (dsa_index_scores)."""
    _need_gpu(q, k, w, q_pos, k_scale, kv_len)
    S, n_q, H, D = q.shape
    n_units = k.shape[1]
    if out is None:
        out = torch.empty((S, n_q, n_units), device=q.device, dtype=torch.float32)
    d = IndexDesc(_ptr(q.contiguous()), _ptr(k.contiguous()), _ptr(k_scale), _ptr(w.contiguous()),
                  _ptr(_i32c(q_pos)), _ptr(_i32c(kv_len)), _dt(q), _dt(k), S, n_q, H, D, n_units,
                  c, int(hadamard_q))
    _check(lib().dsa_index_scores(ctypes.byref(d), _ptr(out), _stream()))
    return out


# ------------------------------------------------------------------- top-k --

def _topk_desc(S, n_q, n_units, q_pos, kv_len, top_k, c, n_sink):
    return TopkDesc(_ptr(_i32c(q_pos)), _ptr(_i32c(kv_len)), S, n_q, n_units, top_k, c, n_sink, 0)


def topk(scores, q_pos, top_k: int, *, c: int = 1, n_sink: int = 0, kv_len=None, out=None):
    """Selected unit ids [S, n_q, top_k // c] int32, ascending, -1 padded (dsa_topk)."""
    _need_gpu(scores, q_pos, kv_len)
    S, n_q, n_units = scores.shape
    if out is None:
        out = torch.empty((S, n_q, top_k // c), device=scores.device, dtype=torch.int32)
    d = _topk_desc(S, n_q, n_units, q_pos, kv_len, top_k, c, n_sink)
    nbytes = lib().dsa_topk_workspace_bytes(ctypes.byref(d))
    ws = torch.empty(max(nbytes, 1), device=scores.device, dtype=torch.uint8)
    _check(lib().dsa_topk(_ptr(scores.contiguous()), ctypes.byref(d), _ptr(out), _ptr(ws), nbytes, _stream()))
    return out


def topk_noalloc(scores, q_pos, top_k: int, *, c: int = 1, n_sink: int = 0, kv_len=None, out=None):
    """dsa_topk on the library's static device scratch (dsa_topk_noalloc):
    allocates nothing on the device when `out` is given.  Calls that overlap
    on one GPU race on the shared scratch."""
    _need_gpu(scores, q_pos, kv_len)
    S, n_q, n_units = scores.shape
    if out is None:
        out = torch.empty((S, n_q, top_k // c), device=scores.device, dtype=torch.int32)
    d = _topk_desc(S, n_q, n_units, q_pos, kv_len, top_k, c, n_sink)
    _check(lib().dsa_topk_noalloc(_ptr(scores.contiguous()), ctypes.byref(d), _ptr(out), _stream()))
    return out


# -------------------------------------------------------------- block pool --

def block_pool(k_raw, c: int, out=None):
    """Mean of every complete block of c raw key rows: [S, n_kv // c, D] f32."""
    _need_gpu(k_raw)
    S, n_kv, D = k_raw.shape
    if out is None:
        out = torch.empty((S, n_kv // c, D), device=k_raw.device, dtype=torch.float32)
    _check(lib().dsa_block_pool(_ptr(k_raw.contiguous()), _dt(k_raw), S, n_kv, D, c, _ptr(out), _stream()))
    return out


def block_pool_update(k_raw, c: int, pooled, from_block, *, kv_len=None):
    """Re-pools, in place, the blocks from_block[s] <= b < min(kv_len[s], n_kv) // c
    of each sequence's persistent pooled keys [S, n_kv // c, D] f32
    (dsa_block_pool_update); every other block is left as it is."""
    _need_gpu(k_raw, pooled, from_block, kv_len)
    S, n_kv, D = k_raw.shape
    if not pooled.is_contiguous() or tuple(pooled.shape) != (S, n_kv // c, D) or pooled.dtype != torch.float32:
        raise DsaError("pooled must be a contiguous [S, n_kv // c, D] float32 tensor")
    _check(lib().dsa_block_pool_update(_ptr(k_raw.contiguous()), _dt(k_raw), S, n_kv, D, c, _ptr(_i32c(from_block)),
                                       _ptr(_i32c(kv_len)), _ptr(pooled), _stream()))
    return pooled


# ------------------------------------------------------ indexer-key cache --

def index_key_write(k_new, cache, *, dst_row=None, cache_scale=None, hadamard: bool = False):
    """Rotates (hadamard=True) and stores new indexer keys [S, n_new, 128] in
    the cache [S, n_cache, 128] (f16, bf16 or float8_e4m3fn with cache_scale
    [S, n_cache] f32) at rows dst_row [S, n_new] int32 (None: rows 0 ..
    n_new - 1); rows outside the cache are skipped (dsa_index_key_write)."""
    _need_gpu(k_new, cache, cache_scale, dst_row)
    if not cache.is_contiguous() or (cache_scale is not None and not cache_scale.is_contiguous()):
        raise DsaError("the key cache and its scales must be contiguous")
    S, n_new, D = k_new.shape
    if cache.dim() != 3 or cache.shape[0] != S or cache.shape[2] != D:
        raise DsaError("cache must be [S, n_cache, D] with the keys' S and D")
    if cache_scale is not None and tuple(cache_scale.shape) != tuple(cache.shape[:2]):
        raise DsaError("cache_scale must be [S, n_cache]")
    if dst_row is not None and tuple(dst_row.shape) != (S, n_new):
        raise DsaError("dst_row must be [S, n_new]")
    _check(lib().dsa_index_key_write(_ptr(k_new.contiguous()), _dt(k_new), S, n_new, D, _ptr(_i32c(dst_row)),
                                     int(hadamard), _ptr(cache), _dt(cache), _ptr(cache_scale), cache.shape[1],
                                     _stream()))
    return cache


# --------------------------------------------------------------- attention --

def _strides(t):
    """(seq, token, head) element strides of a [S, n_kv, H, D] tensor view."""
    if t.stride(3) != 1:
        raise DsaError("the last dimension of K/V must be contiguous")
    return t.stride(0), t.stride(1), t.stride(2)


def _kv_format(K, kv_scale):
    """(kv_format, scale pointer): q8_0 when the latent rows are int8 codes."""
    if K.dtype == torch.int8:
        if kv_scale is None or kv_scale.dtype != torch.float16 or not kv_scale.is_contiguous():
            raise DsaError("q8_0 latent rows need kv_scale: contiguous f16 [S, n_kv, Dk // 32]")
        return Q8_0, _ptr(kv_scale)
    if kv_scale is not None:
        raise DsaError("kv_scale is only for int8 (q8_0) latent rows")
    return 0, None


def _attn_desc(Q, K, V, q_pos, kv_len, k_sel, c, scale, o_dtype, kv_scale=None):
    S, n_q, Hq, Dk = Q.shape
    _, n_kv, Hkv, _ = K.shape
    Dv = V.shape[3]
    ks, vs = _strides(K), _strides(V)
    fmt, sc = _kv_format(K, kv_scale)
    return AttnDesc(_ptr(Q), _ptr(K), _ptr(V), ks[0], ks[1], ks[2], vs[0], vs[1], vs[2],
                    _ptr(_i32c(q_pos)), _ptr(_i32c(kv_len)), _dt(Q), DTYPES[o_dtype],
                    S, n_q, Hq, Hkv, Dk, Dv, n_kv, k_sel, c, 0.0 if scale is None else float(scale), fmt, sc)


def sparse_attn(Q, K, V, q_pos, idx=None, *, c: int = 1, kv_len=None, scale=None,
                o_dtype=torch.float32, out=None, kv_scale=None):
    """Attention over the selected tokens (idx None = dense causal): [S, n_q, Hq, Dv].
    q8_0 latent rows: K int8 codes [S, n_kv, 1, 576], V = K[..., :512], and
    kv_scale f16 [S, n_kv, 18]."""
    _need_gpu(Q, K, V, q_pos, idx, kv_len, kv_scale)
    Q = Q.contiguous()
    S, n_q, Hq, _ = Q.shape
    Dv = V.shape[3]
    k_sel = 0 if idx is None else idx.shape[2]
    if idx is not None:
        idx = _i32c(idx.contiguous())
    d = _attn_desc(Q, K, V, q_pos, kv_len, k_sel, c, scale, o_dtype, kv_scale)
    if out is None:
        out = torch.empty((S, n_q, Hq, Dv), device=Q.device, dtype=o_dtype)
    nbytes = lib().dsa_sparse_attn_workspace_bytes(ctypes.byref(d), int(idx is None))
    ws = torch.empty(max(nbytes, 1), device=Q.device, dtype=torch.uint8)
    _check(lib().dsa_sparse_attn(ctypes.byref(d), _ptr(idx), _ptr(out), _ptr(ws), nbytes, _stream()))
    return out


# ----------------------------------------------------------------- forward --

class Event:
    """A HIP event created through the library (for phase timing)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().dsa_event_create(ctypes.byref(h)))
        self.handle = h

    def record(self):
        _check(lib().dsa_event_record(self.handle, _stream()))

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float()
        _check(lib().dsa_event_elapsed_ms(self.handle, end.handle, ctypes.byref(ms)))
        return ms.value

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dsa_event_destroy(self.handle)


def _forward_desc(Q, K, V, q_idx, k_idx, w, top_k, c, q_pos, k_scale, n_sink, scale, hadamard_q,
                  kv_len, out, idx_out, scores_out, events_arr, kv_scale=None):
    S, n_q, Hq, Dk = Q.shape
    _, n_kv, Hkv, _ = K.shape
    Dv = V.shape[3]
    H, D = q_idx.shape[2], q_idx.shape[3]
    ks, vs = _strides(K), _strides(V)
    fmt, sc = _kv_format(K, kv_scale)
    return ForwardDesc(_ptr(q_idx), _ptr(k_idx), _ptr(k_scale), _ptr(w), _dt(q_idx), _dt(k_idx), H, D,
                       top_k, c, n_sink, int(hadamard_q), _ptr(Q), _ptr(K), _ptr(V),
                       ks[0], ks[1], ks[2], vs[0], vs[1], vs[2], _dt(Q), DTYPES[out.dtype], Hq, Hkv, Dk, Dv,
                       0.0 if scale is None else float(scale), fmt, S, n_q, n_kv,
                       _ptr(_i32c(q_pos)), _ptr(_i32c(kv_len)), _ptr(out), _ptr(idx_out), _ptr(scores_out),
                       None if events_arr is None else ctypes.cast(events_arr, ctypes.c_void_p), sc)


def forward_workspace_bytes(Q, K, V, q_idx, k_idx, w, top_k, compress_ratio, q_pos, *, k_scale=None,
                            n_sink=0, scale=None, hadamard_q=False, kv_len=None, o_dtype=torch.float32,
                            return_idx=False, return_scores=False, kv_scale=None) -> int:
    S, n_q, Hq, _ = Q.shape
    out = torch.empty(0, dtype=o_dtype)
    dummy = ctypes.c_void_p(16)
    d = _forward_desc(Q, K, V, q_idx, k_idx, w, top_k, compress_ratio, q_pos, k_scale, n_sink, scale,
                      hadamard_q, kv_len, out, None, None, None, kv_scale)
    d.out = dummy
    if return_idx:
        d.idx_out = dummy
    if return_scores:
        d.scores_out = dummy
    return int(lib().dsa_forward_workspace_bytes(ctypes.byref(d)))


def forward(Q, K, V, q_idx, k_idx, w, top_k: int, compress_ratio: int, q_pos, *, k_scale=None,
            n_sink: int = 0, scale=None, hadamard_q: bool = False, kv_len=None, out=None,
            o_dtype=torch.float32, return_idx: bool = False, return_scores: bool = False,
            workspace: Optional[torch.Tensor] = None, phase_events: Optional[Sequence[Event]] = None,
            kv_scale=None):
    """The whole path (dsa_forward): O [S, n_q, Hq, Dv], plus idx / scores if asked.
    q8_0 latent rows as in sparse_attn (K int8 codes, kv_scale f16)."""
    _need_gpu(Q, K, V, q_idx, k_idx, w, q_pos, k_scale, kv_len, kv_scale)
    S, n_q, Hq, _ = Q.shape
    Dv = V.shape[3]
    n_kv = K.shape[1]
    c = compress_ratio
    n_units = n_kv // c if c > 1 else n_kv
    Q, q_idx, k_idx, w = Q.contiguous(), q_idx.contiguous(), k_idx.contiguous(), w.contiguous()
    if out is None:
        out = torch.empty((S, n_q, Hq, Dv), device=Q.device, dtype=o_dtype)
    idx_out = torch.empty((S, n_q, top_k // c), device=Q.device, dtype=torch.int32) if return_idx else None
    scores_out = (torch.empty((S, n_q, max(n_units, 1)), device=Q.device, dtype=torch.float32)
                  if return_scores else None)
    events_arr = None
    if phase_events is not None:
        events_arr = (ctypes.c_void_p * 5)(*[None if e is None else e.handle.value for e in phase_events])
    d = _forward_desc(Q, K, V, q_idx, k_idx, w, top_k, c, q_pos, k_scale, n_sink, scale, hadamard_q,
                      kv_len, out, idx_out, scores_out, events_arr, kv_scale)
    nbytes = int(lib().dsa_forward_workspace_bytes(ctypes.byref(d)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), device=Q.device, dtype=torch.uint8)
    _check(lib().dsa_forward(ctypes.byref(d), _ptr(workspace), nbytes, _stream()))
    res = [out]
    if return_idx:
        res.append(idx_out)
    if return_scores:
        res.append(scores_out)
    return res[0] if len(res) == 1 else tuple(res)


# --------------------------------------------------------------- IndexShare --

def index_share_source(layer: int) -> int:
    """The layer whose selection `layer` attends over (dsa_index_share_source)."""
    r = lib().dsa_index_share_source(layer)
    if r < 0:
        _check(r)
    return r


def forward_layers(layers, top_k: int, compress_ratio: int, q_pos, *, n_sink: int = 0, hadamard_q: bool = False,
                   kv_len=None, outs=None):
    """A stack of DSA attention layers under IndexShare: full layers run
    dsa_forward and keep their index rows, shared layers run dsa_sparse_attn
    over the rows of their source layer.  layers[il] is a dict with Q, K, V,
    q_idx, k_idx, w (optional k_scale, scale).  Returns (outputs, index rows)."""
    res, idxs = [], []
    for il, L in enumerate(layers):
        src = index_share_source(il)
        out = None if outs is None else outs[il]
        if src == il:
            O, idx = forward(L["Q"], L["K"], L["V"], L["q_idx"], L["k_idx"], L["w"], top_k, compress_ratio, q_pos,
                             k_scale=L.get("k_scale"), n_sink=n_sink, scale=L.get("scale"), hadamard_q=hadamard_q,
                             kv_len=kv_len, out=out, return_idx=True)
        else:
            idx = idxs[src]
            O = sparse_attn(L["Q"], L["K"], L["V"], q_pos, idx, c=compress_ratio, kv_len=kv_len,
                            scale=L.get("scale"), out=out)
        res.append(O)
        idxs.append(idx)
    return res, idxs

