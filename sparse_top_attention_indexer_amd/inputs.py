"""Seeded synthetic workloads for the DSA hot path.

This module only draws random numbers, casts them to the stored element types
and lays them out; it holds none of the method's arithmetic.  The same tensors
feed the HIP library and the CPU oracle.

Five workloads, each with the shapes, value distributions and structure of
the sparse-attention configurations this library is built for:

  1 tiny prefill      1 x 256 causal, indexer 4 heads x 128 fp32, w ~ U(0,1),
                      top_k 64 (and 256); attention 4 heads x 64 fp32, scale 1/8
  2 DSA prefill       1 x 4096 causal, indexer 64 x 128 bf16, w ~ N(0,1)/8,
                      top_k 2048; MLA attention 128 heads over a 576-wide
                      latent (V = its first 512 columns), bf16
  3 batched decode    32 sequences x 1 query against 32768 cached keys; fp16
                      indexer-key cache; top_k 2048; one attention-sink key
  4 QSA prefill chunk 2048 queries at positions 14336..16383 over 16384 keys;
                      raw bf16 keys pooled in blocks of 64; top_k 4096 (64
                      blocks); GQA 32 query / 4 KV heads x 128 bf16
  5 long decode       8 sequences x 131072 cached keys; index keys stored
                      Walsh-Hadamard-rotated as fp8 e4m3fn with a per-row fp32
                      scale; queries rotated in-kernel; 1 % of token rows x 8

Storage of the fp8 index keys (the cache-write step, which precedes the hot
path): a Walsh-Hadamard rotation is orthonormal, so a rotated i.i.d. N(0,1)
row is again i.i.d. N(0,1); the stored rotated rows are therefore drawn
directly from N(0,1) (x 8 on outlier rows), then each row is scaled by
amax/448 and cast with torch's float8_e4m3fn conversion.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    S: int                 # sequences
    n_q: int               # queries per sequence
    n_kv: int              # cached keys per sequence
    q_pos0: int            # position of the first query (queries are consecutive)
    H: int                 # indexer heads
    D: int                 # indexer dim
    q_dtype: torch.dtype   # indexer query dtype
    k_dtype: torch.dtype   # indexer key storage dtype (fp8 => per-row scale)
    w_kind: str            # "uniform" (U(0,1)) or "normal" (N(0,1) * w_std)
    w_std: float
    top_k: int
    c: int                 # compress ratio (1 = token mode)
    n_sink: int
    hadamard_q: bool
    attn: str              # "f32" | "mla" | "gqa"
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    a_dtype: torch.dtype   # attention Q/K/V dtype
    scale: float           # attention softmax scale
    outlier_frac: float = 0.0
    seed: int = 1000

    @property
    def k_out(self) -> int:
        return self.top_k // self.c

    @property
    def rows(self) -> int:
        return self.S * self.n_q


def preset(n: int) -> Workload:
    """Full-size workload n (1..5)."""
    if n == 1:
        return Workload("tiny_prefill_256", 1, 256, 256, 0, 4, 128, torch.float32,
                        torch.float32, "uniform", 1.0, 64, 1, 0, False, "f32",
                        4, 4, 64, 64, torch.float32, 1.0 / 8.0, seed=1001)
    if n == 2:
        return Workload("dsa_prefill_4096_mla", 1, 4096, 4096, 0, 64, 128, torch.bfloat16,
                        torch.bfloat16, "normal", 1.0 / 8.0, 2048, 1, 0, False, "mla",
                        128, 1, 576, 512, torch.bfloat16, 1.0 / math.sqrt(576), seed=1002)
    if n == 3:
        return Workload("batched_decode_32x32768_mla", 32, 1, 32768, 32767, 64, 128,
                        torch.bfloat16, torch.float16, "normal", 1.0 / 8.0, 2048, 1, 1,
                        False, "mla", 128, 1, 576, 512, torch.bfloat16,
                        1.0 / math.sqrt(576), seed=1003)
    if n == 4:
        return Workload("qsa_chunk_2048_of_16384_gqa", 1, 2048, 16384, 14336, 16, 128,
                        torch.bfloat16, torch.bfloat16, "normal", 1.0 / 4.0, 4096, 64, 0,
                        False, "gqa", 32, 4, 128, 128, torch.bfloat16,
                        1.0 / math.sqrt(128), seed=1004)
    if n == 5:
        return Workload("long_decode_8x131072_fp8_mla", 8, 1, 131072, 131071, 64, 128,
                        torch.bfloat16, torch.float8_e4m3fn, "normal", 1.0 / 8.0, 2048, 1,
                        0, True, "mla", 128, 1, 576, 512, torch.bfloat16,
                        1.0 / math.sqrt(576), outlier_frac=0.01, seed=1005)
    raise ValueError(n)


def mini(n: int) -> Workload:
    """Reduced workload n: same structure, sizes that span several tiles and a
    ragged tail but that the CPU oracle finishes in seconds."""
    w = preset(n)
    if n == 1:
        return w
    if n == 2:
        return replace(w, name="dsa_prefill_mini", n_q=700, n_kv=700, top_k=256)
    if n == 3:
        return replace(w, name="batched_decode_mini", S=5, n_kv=3001, q_pos0=3000, top_k=512)
    if n == 4:
        return replace(w, name="qsa_chunk_mini", n_q=300, n_kv=2000, q_pos0=1700, c=16,
                       top_k=512)
    if n == 5:
        return replace(w, name="long_decode_mini", S=3, n_kv=5003, q_pos0=5002, top_k=512)
    raise ValueError(n)


def _randn(g, shape, device, dtype=torch.float32):
    return torch.randn(shape, generator=g, device=device, dtype=dtype)


def generate(wl: Workload, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw every input of workload wl on `device` in a fixed order.

    Returns a dict with
      q_idx [S, n_q, H, D]      indexer queries (wl.q_dtype)
      k_idx [S, n_kv, D]        indexer keys: token keys (c == 1) or raw keys to
                                pool (c > 1), stored as wl.k_dtype
      k_scale [S, n_kv] f32     per-row dequantisation scale (fp8 keys) or None
      w [S, n_q, H] f32         head weights
      q_pos [S, n_q] int32      query positions
      kv_len [S] int32          cached keys per sequence
      Q [S, n_q, Hq, Dk]        attention queries
      K [S, n_kv, Hkv, Dk]      attention keys (MLA: the latent rows)
      V [S, n_kv, Hkv, Dv]      attention values (MLA: a view of K[..., :Dv])
    """
    seed = wl.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    S, n_q, n_kv, H, D = wl.S, wl.n_q, wl.n_kv, wl.H, wl.D

    out: dict = {"wl": wl}
    out["q_idx"] = _randn(g, (S, n_q, H, D), device).to(wl.q_dtype)

    # outlier token rows (shared by the index keys and the attention rows)
    n_out = int(round(wl.outlier_frac * n_kv))
    row_gain = torch.ones(S, n_kv, device=device)
    if n_out > 0:
        for s in range(S):
            rows = torch.randperm(n_kv, generator=g, device=device)[:n_out]
            row_gain[s, rows] = 8.0

    k = _randn(g, (S, n_kv, D), device) * row_gain[..., None]
    if wl.k_dtype == torch.float8_e4m3fn:
        amax = k.abs().amax(dim=-1).clamp_min(1e-30)
        scale = amax / 448.0
        codes = (k / scale[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        out["k_idx"], out["k_scale"] = codes, scale.to(torch.float32).contiguous()
    else:
        out["k_idx"], out["k_scale"] = k.to(wl.k_dtype), None

    if wl.w_kind == "uniform":
        w = torch.rand((S, n_q, H), generator=g, device=device)
    else:
        w = _randn(g, (S, n_q, H), device) * wl.w_std
    out["w"] = w.to(torch.float32).contiguous()

    pos = torch.arange(wl.q_pos0, wl.q_pos0 + n_q, device=device, dtype=torch.int32)
    out["q_pos"] = pos.expand(S, n_q).contiguous()
    out["kv_len"] = torch.full((S,), n_kv, device=device, dtype=torch.int32)

    out["Q"] = _randn(g, (S, n_q, wl.Hq, wl.Dk), device).to(wl.a_dtype)
    if wl.attn == "mla":
        lat = (_randn(g, (S, n_kv, wl.Dk), device) * row_gain[..., None]).to(wl.a_dtype)
        out["K"] = lat.view(S, n_kv, 1, wl.Dk)
        out["V"] = out["K"][..., :wl.Dv]          # aliases the latent rows
    else:
        out["K"] = (_randn(g, (S, n_kv, wl.Hkv, wl.Dk), device) *
                    row_gain[..., None, None]).to(wl.a_dtype)
        out["V"] = (_randn(g, (S, n_kv, wl.Hkv, wl.Dv), device) *
                    row_gain[..., None, None]).to(wl.a_dtype)
    return out


def key_write_batch(S: int, n_new: int, n_cache: int, k_dtype=torch.bfloat16, seed: int = 2000,
                    outlier_frac: float = 0.01, zero_rows: int = 1, skipped: int = 2,
                    device="cpu") -> dict:
    """New raw indexer keys for the cache-write step and where they go.

    k_new [S, n_new, 128] ~ N(0,1) in k_dtype, with a seeded share of rows x 8
    (the long-decode workload's outliers) and `zero_rows` all-zero rows per
    sequence.  dst_row [S, n_new] int32: distinct cache rows drawn at random
    per sequence, except that `skipped` entries per sequence point outside the
    cache (-1, n_cache) and must leave it untouched.  Needs n_new <= n_cache.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn((S, n_new, 128), generator=g)
    out = torch.rand((S, n_new), generator=g) < outlier_frac
    k[out] *= 8.0
    for s in range(S):
        k[s, :min(zero_rows, n_new)] = 0.0
    dst = torch.stack([torch.randperm(n_cache, generator=g)[:n_new] for _ in range(S)]).to(torch.int32)
    for s in range(S):
        for j in range(min(skipped, n_new)):
            dst[s, n_new - 1 - j] = -1 if j % 2 == 0 else n_cache
    return {"k_new": k.to(k_dtype).to(device), "dst_row": dst.to(device)}


def indexer_queries(S: int, n_q: int, H: int = 64, seed: int = 2007) -> dict:
    """Indexer queries [S, n_q, H, 128] bf16 ~ N(0,1) and head weights
    [S, n_q, H] f32 ~ N(0,1)/sqrt(H), for scoring a written key cache."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((S, n_q, H, 128), generator=g).to(torch.bfloat16)
    w = torch.randn((S, n_q, H), generator=g) / math.sqrt(H)
    return {"q_idx": q, "w": w}


def raw_key_batch(S: int, n_kv: int, D: int = 128, dtype=torch.bfloat16, seed: int = 3000) -> torch.Tensor:
    """Raw (unpooled) indexer keys [S, n_kv, D] ~ N(0,1) in dtype, as the
    block-pooled workload stores them."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((S, n_kv, D), generator=g).to(dtype)


def q8_0_latent(latent: torch.Tensor):
    """The MLA latent rows [S, n_kv, 1, D] (D a multiple of 32) cached as q8_0,
    the quantised latent cache type: codes int8 [S, n_kv, 1, D] and scales
    f16 [S, n_kv, D / 32], one per block of 32 values (scale = f16(max |x| /
    127), code = x / scale rounded half away from zero).  This is the cache
    write that precedes attention; the values come from the seeded latent."""
    S, n, h, D = latent.shape
    x = latent.float().reshape(S, n, D // 32, 32)
    scale = (x.abs().amax(dim=-1) / 127.0).to(torch.float16)
    s32 = scale.float().unsqueeze(-1)
    q = torch.where(s32 > 0, x / torch.where(s32 > 0, s32, torch.ones_like(s32)), torch.zeros_like(x))
    codes = (torch.sign(q) * torch.floor(q.abs() + 0.5)).clamp(-127, 127).to(torch.int8)
    return codes.reshape(S, n, 1, D).contiguous(), scale.contiguous()
