"""Benchmark of the DSA hot path on one MI355X.

One step = one dsa_forward call over the whole batch of the workload: indexer
scores -> top-k -> sparse attention (block pooling first in block mode).
Inputs are seeded synthetic tensors already resident in HBM.  Prints one JSON
line.  The headline workload is the 4096-token DSA prefill (128-head MLA
attention over a 576-wide latent, 64-head bf16 indexer, top_k 2048); the
line's "configs" object times the other four workloads with the same
protocol (tiny prefill, batched decode, block-pooled chunk, long decode).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 1..5]
                    [--no-cpu-baseline] [--no-next-rows] [--next-rows-only] [--no-flush]
                    [--headline-only] [--calib-copy]

--config n makes workload n the headline and times nothing else.  Beside the
hot path it times the indexer-key cache write (rotate + fp8 quantise) at the
long-decode cache shape, the incremental block pooling of one micro-batch,
an 8-layer IndexShare decode stack, and decode attention over q8_0 latent
rows against bf16 ones, reported under "next_rows".
"""

import argparse
import json
import math
import os
import sys
import time

# The oracle's BLAS pool: every host core the run may use, set before numpy
# loads its BLAS (an explicit OMP_NUM_THREADS, as on a shared host, is kept).
_BLAS_THREADS = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count() or 1)
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, _BLAS_THREADS)

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
CSRC = os.path.join(ROOT, "sparse_top_attention_indexer_amd")
PROFILES = os.path.join(ROOT, "profiles")
# dense MFMA peaks; f32 is the vector (VALU) peak of code built without
# packed-FP32 instructions: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
PEAK = {"bf16": 2.5e15, "f16": 2.5e15, "fp8": 5.0e15, "f32": 78.6e12}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="time only workload 1..5 as the headline (default: workload 2, plus the others)")
    ap.add_argument("--headline-only", action="store_true", help="do not time the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not evict the caches before each timed step (warm-cache timing by wall clock)")
    ap.add_argument("--next-rows-only", action="store_true",
                    help="only the rows measured beside the hot path, as one JSON object (for kernel traces)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the rows measured beside the hot path (key-cache write, incremental pooling, IndexShare)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run one 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------ kernel names, traffic

def score_kernel_name(wl):
    """The score kernel the library picks for this workload (its launch rules)."""
    import torch
    n_units = wl.n_kv // wl.c
    rows = wl.S * wl.n_q
    if wl.k_dtype == torch.float32 and wl.q_dtype == torch.float32:
        return "score_valu_kernel"
    if wl.c > 1:   # pooled block keys are f32
        return "score_tiled_kernel" if wl.n_q % 4 == 0 else "score_mfma_kernel"
    multiblock = n_units > 16384 or (rows < 128 and n_units > 4096)
    if multiblock and wl.k_dtype != torch.float32:
        return "score_stream_kernel"
    if wl.k_dtype in (torch.bfloat16, torch.float16, torch.float32) and wl.n_q % 4 == 0:
        return "score_tiled_kernel"
    return "score_mfma_kernel"


def attn_kernel_name(wl):
    """The attention kernel the library picks for workload wl: GQA calls with
    8+ queries a sequence in dense mode or with blocks of a multiple of 32
    tokens run over query tiles."""
    if wl.attn == "gqa":
        tiled = wl.n_q >= 8 and (wl.c > 1 and wl.c % 32 == 0) and 16 % (wl.Hq // wl.Hkv) == 0
        return "attn_gqa_tile_kernel" if tiled else "attn_gqa_kernel"
    return {"mla": "attn_mla_kernel", "f32": "attn_f32_kernel"}[wl.attn]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record (calibrated by a copy of known
    size), or None when there is none or the kernel's sources changed since."""
    import glob
    import hashlib
    for f in sorted(glob.glob(os.path.join(PROFILES, "*_traffic.md"))):
        for line in open(f):
            if not line.startswith("traffic-record: "):
                continue
            rec = json.loads(line[len("traffic-record: "):])
            if rec["workload"] != workload or rec["kernel"] != kernel:
                continue
            h = hashlib.sha256()
            for src in rec["sources"]:
                with open(os.path.join(CSRC, src), "rb") as fh:
                    h.update(fh.read())
            return rec["bytes"] if h.hexdigest() == rec["source_sha256"] else None
    return None


# ------------------------------------------------------------ algorithmic work

def work_model(wl, q_pos, kv_len):
    """Per-phase algorithmic flops and HBM bytes of one step (what the method
    must compute and move), from the positions and sizes of the workload."""
    qp = q_pos.astype(np.int64)
    kv = np.repeat(kv_len.astype(np.int64)[:, None], wl.n_q, axis=1)
    n_vis = np.clip(np.minimum(qp + 1, kv), 0, None)                 # visible tokens per query
    units = n_vis // wl.c                                             # visible scored units
    k_out = wl.top_k // wl.c
    if wl.c > 1:
        sel = np.minimum(units, k_out) * wl.c + (n_vis - units * wl.c)  # blocks + tail
    else:
        sel = np.minimum(units, k_out)
    pairs_score = int(units.sum())
    pairs_attn = int(sel.sum())
    esz = {"torch.bfloat16": 2, "torch.float16": 2, "torch.float32": 4, "torch.float8_e4m3fn": 1}
    kb = esz[str(wl.k_dtype)]
    qb = esz[str(wl.q_dtype)]
    ab = esz[str(wl.a_dtype)]
    rows = wl.S * wl.n_q
    n_units_row = wl.n_kv // wl.c
    d = {}
    # S1 block pooling: read raw keys, write pooled keys
    d["pool"] = dict(flops=0, bytes=(wl.S * wl.n_kv * wl.D * kb + wl.S * n_units_row * wl.D * 4) if wl.c > 1 else 0)
    # S2 scores: one dot of D per head per visible unit; q, keys (+scales), w read, scores written
    key_bytes = wl.S * n_units_row * wl.D * (4 if wl.c > 1 else kb)
    if wl.k_dtype.is_floating_point and kb == 1:
        key_bytes += wl.S * n_units_row * 4
    d["scores"] = dict(flops=2 * pairs_score * wl.H * wl.D,
                       bytes=rows * wl.H * wl.D * qb + key_bytes + rows * wl.H * 4 + pairs_score * 4)
    # S3 top-k: visible scores read, index rows written
    d["topk"] = dict(flops=0, bytes=pairs_score * 4 + rows * k_out * 4)
    # S5 attention: q.k over Dk and p.v over Dv per head per selected token; Q read, the
    # selected K/V rows read (each distinct row once), O written
    if wl.attn == "mla":
        kv_row_bytes = wl.Dk * ab
        distinct = wl.S * wl.n_kv * kv_row_bytes if wl.n_q > 1 else pairs_attn * kv_row_bytes
    else:
        kv_row_bytes = wl.Hkv * (wl.Dk + wl.Dv) * ab
        distinct = wl.S * wl.n_kv * kv_row_bytes if wl.n_q > 1 else pairs_attn * kv_row_bytes
    d["attn"] = dict(flops=2 * pairs_attn * wl.Hq * (wl.Dk + wl.Dv),
                     bytes=rows * wl.Hq * wl.Dk * ab + distinct + rows * wl.Hq * wl.Dv * 4)
    return d, pairs_score, pairs_attn


def compute_dtype(wl):
    if wl.a_dtype.__repr__() == "torch.float32":
        return "f32"
    return "bf16"


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline(wl, x, budget_s):
    """Times the CPU oracle on a bounded sample of query rows of the same
    workload (rows evenly spread over the batch, so the causal cost mix is
    kept), and scales to query tokens/s."""
    import torch
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:   # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    f = O.to_f64
    rows = [(s, i) for s in range(wl.S) for i in range(wl.n_q)]
    # bit-reversed order: every prefix of it is spread evenly over the batch
    nb = max(1, (len(rows) - 1).bit_length())
    order = sorted(range(len(rows)), key=lambda r: int(format(r, f"0{nb}b")[::-1], 2))
    sample = [rows[r] for r in order]
    # inputs the sampled rows read, converted once outside the timed region
    k_idx = [f(x["k_idx"][s:s + 1]) for s in range(wl.S)]
    k_scale = [None if x["k_scale"] is None else f(x["k_scale"][s:s + 1]) for s in range(wl.S)]
    K = [f(x["K"][s:s + 1]) for s in range(wl.S)]
    V = [f(x["V"][s:s + 1]) for s in range(wl.S)]
    kv = x["kv_len"].cpu().numpy()
    done, t_total, scored = 0, 0.0, 0
    kvn = x["kv_len"].cpu().numpy()
    for s, i in sample:
        qi = f(x["q_idx"][s:s + 1, i:i + 1])
        w = f(x["w"][s:s + 1, i:i + 1])
        Q = f(x["Q"][s:s + 1, i:i + 1])
        qp = x["q_pos"][s:s + 1, i:i + 1].cpu().numpy()
        t0 = time.perf_counter()
        O.forward(Q, K[s], V[s], qi, k_idx[s], w, wl.top_k, wl.c, qp, kv[s:s + 1], k_scale[s],
                  wl.n_sink if wl.c == 1 else 0, wl.scale, wl.hadamard_q)
        t_total += time.perf_counter() - t0
        done += 1
        n_vis = max(0, min(int(qp[0, 0]) + 1, int(kvn[s]), wl.n_kv))
        scored += n_vis // wl.c
        if t_total > budget_s and done >= 4:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": done / t_total, "unit": "query tokens/s", "keys_scored_per_s": scored / t_total,
            "cores": threads, "host_cores": os.cpu_count(), "blas_threads": threads,
            "cpu_model": model, "kind": "oracle",
            "sample": f"{done} of {len(rows)} query rows of the {wl.name} batch, taken in bit-reversed order "
                      f"(evenly spread), numpy float64 oracle, {t_total:.1f} s"}


# ------------------------------------------------ next row: key cache write

def key_write_row(dsa, inputs, torch, steps):
    """The indexer-key cache write at the long-decode cache shape: 8 x 131072
    new bf16 keys rotated and stored as fp8 e4m3fn + f32 row scales in one
    call.  Timed with HIP events on the stream the binding launches on; HBM
    roofline on algorithmic bytes (each key row read once, its codes and
    scale written once)."""
    S, n = 8, 131072
    b = inputs.key_write_batch(S, n, n, torch.bfloat16, seed=2005, skipped=0, device="cuda")
    cache = torch.empty((S, n, 128), dtype=torch.float8_e4m3fn, device="cuda")
    scale = torch.empty((S, n), dtype=torch.float32, device="cuda")

    def run():
        dsa.index_key_write(b["k_new"], cache, cache_scale=scale, hadamard=True)

    for _ in range(3):
        run()
    ev = [dsa.Event() for _ in range(steps + 1)]
    ev[0].record()
    for k in range(steps):
        run()
        ev[k + 1].record()
    torch.cuda.synchronize()
    ms = sum(ev[k].elapsed_ms(ev[k + 1]) for k in range(steps)) / steps
    per_row = 128 * 2 + 128 + 4
    by = S * n * per_row
    name = "index_key_write_8x131072_bf16_to_fp8_rotated"
    return {"workload": name, "kernel": "key_write_kernel",
            "ms": round(ms, 5), "rows_per_s": S * n / (ms * 1e-3), "bytes_per_row": per_row,
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": by / (ms * 1e-3) / PEAK_HBM, "traffic": measured_traffic(name, "key_write_kernel")}}


# ------------------------------------------- next row: incremental pooling

def pool_update_row(dsa, inputs, torch, steps):
    """Incremental block pooling at the block-pooled workload's shape: 16384
    bf16 raw keys, blocks of 64; one micro-batch of 2048 new tokens re-pools
    its 32 blocks into the persistent pooled keys, against a one-shot pool
    of all 256 blocks.  HIP events on the launch stream; HBM roofline on
    algorithmic bytes (raw rows read once, pooled f32 rows written once)."""
    n, c = 16384, 64
    k = inputs.raw_key_batch(1, n, seed=3004).to("cuda")
    pooled = dsa.block_pool(k, c)
    first = torch.tensor([(n - 2048) // c], dtype=torch.int32, device="cuda")

    def timed(fn):
        # the calls take a few microseconds on the GPU, less than the binding
        # takes to issue one: queue them behind a ~1 ms spin kernel, so that
        # they run back to back and the events time the GPU, not the host
        for _ in range(3):
            fn()
        ev = [dsa.Event() for _ in range(2)]
        torch.cuda.synchronize()
        torch.cuda._sleep(2_000_000)
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_ms(ev[1]) / steps

    ms_inc = timed(lambda: dsa.block_pool_update(k, c, pooled, first))
    ms_full = timed(lambda: dsa.block_pool(k, c, out=pooled))
    by_inc = 32 * c * 128 * 2 + 32 * 128 * 4
    return {"workload": "block_pool_update_2048_new_of_16384_c64", "kernel": "block_pool_kernel",
            "ms": round(ms_inc, 5), "ms_full_repool": round(ms_full, 5), "blocks": 32, "blocks_full": 256,
            "roofline": {"bound": "hbm", "achieved": by_inc / (ms_inc * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": by_inc / (ms_inc * 1e-3) / PEAK_HBM},
            "note": "one launch of a few microseconds: the time is the launch floor (the full re-pool of 8x the "
                    "blocks takes the same), not HBM"}


# ---------------------------------------------------- next row: IndexShare

def index_share_row(dsa, inputs, torch, steps):
    """An 8-layer stack at the batched-decode shape (32 sequences x 32768
    cached keys, 128-head MLA) under IndexShare (layers 0, 1, 2, 6 select,
    3-5 and 7 reuse the latest full layer's rows), against the same stack with
    every layer selecting on its own.  The layers share one set of inputs
    (the work per layer does not depend on the values); calls are queued
    behind a spin kernel so that the events time the GPU."""
    wl = inputs.preset(3)
    x = inputs.generate(wl, device="cuda")
    layer = {k: x[k] for k in ("Q", "K", "V", "q_idx", "k_idx", "w", "k_scale")}
    layer["scale"] = wl.scale
    n_layers = 8
    layers = [layer] * n_layers
    outs = [torch.empty((wl.S, wl.n_q, wl.Hq, wl.Dv), device="cuda") for _ in range(n_layers)]
    kw = dict(n_sink=wl.n_sink, hadamard_q=wl.hadamard_q, kv_len=x["kv_len"])

    def shared():
        dsa.forward_layers(layers, wl.top_k, wl.c, x["q_pos"], outs=outs, **kw)

    def own():
        for il in range(n_layers):
            dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, wl.c, x["q_pos"],
                        k_scale=x["k_scale"], scale=wl.scale, out=outs[il], **kw)

    def timed(fn):
        for _ in range(2):
            fn()
        ev = [dsa.Event() for _ in range(2)]
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_ms(ev[1]) / steps

    ms_shared, ms_own = timed(shared), timed(own)
    full = sum(1 for il in range(n_layers) if dsa.index_share_source(il) == il)
    return {"workload": "index_share_8_layers_batched_decode_32x32768", "layers": n_layers, "full_layers": full,
            "ms_per_stack": round(ms_shared, 5), "ms_per_stack_all_full": round(ms_own, 5),
            "query_tokens_per_s": wl.S * wl.n_q / (ms_shared * 1e-3), "speedup": round(ms_own / ms_shared, 3)}


# ------------------------------------------------ next row: q8_0 latent rows

def q8_latent_row(dsa, inputs, torch, steps, flush):
    """Decode attention over the latent rows cached as q8_0 against the same
    rows in bf16, at the batched-decode (32 x 32768) and long-decode
    (8 x 131072) shapes: the indexer's top-k of each workload selects the
    rows, then attention alone is timed (dsa_sparse_attn: the gathered tile
    kernel and the split merge), caches flushed before each call, HIP events
    on the launch stream.  Algorithmic bytes: each selected row once (1152
    bytes in bf16; 576 codes + 18 f16 scales = 612 in q8_0), the queries read
    and the f32 outputs written; flops: 2 (576 + 512) per head and row."""
    res = {}
    for n in (3, 5):
        wl = inputs.preset(n)
        x = inputs.generate(wl, device="cuda")
        sc = dsa.index_scores(x["q_idx"], x["k_idx"], x["w"], x["q_pos"], k_scale=x["k_scale"],
                              kv_len=x["kv_len"], hadamard_q=wl.hadamard_q)
        idx = dsa.topk(sc, x["q_pos"], wl.top_k, n_sink=wl.n_sink, kv_len=x["kv_len"])
        del sc
        codes, scales = inputs.q8_0_latent(x["K"])
        out_b = torch.empty((wl.S, wl.n_q, wl.Hq, wl.Dv), device="cuda", dtype=torch.float32)
        out_q = torch.empty_like(out_b)
        kw = dict(kv_len=x["kv_len"], scale=wl.scale)

        def bf16():
            dsa.sparse_attn(x["Q"], x["K"], x["V"], x["q_pos"], idx, out=out_b, **kw)

        def q8():
            dsa.sparse_attn(x["Q"], codes, codes[..., :wl.Dv], x["q_pos"], idx, kv_scale=scales, out=out_q, **kw)

        def timed(fn):
            for _ in range(3):
                fn()
            ev = [(dsa.Event(), dsa.Event()) for _ in range(steps)]
            for a, b in ev:
                if flush is not None:
                    flush.amax()
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            return sum(a.elapsed_ms(b) for a, b in ev) / steps

        ms_b, ms_q = timed(bf16), timed(q8)
        pairs = int((idx >= 0).sum().item())
        io = wl.S * wl.n_q * wl.Hq * (wl.Dk * 2 + wl.Dv * 4)
        by_b, by_q = pairs * 1152 + io, pairs * 612 + io
        fl = 2.0 * pairs * wl.Hq * (wl.Dk + wl.Dv)
        linf = float((out_q - out_b).abs().max() / out_b.abs().max())
        res[wl.name] = {
            "kernel": "attn_mla_q8_kernel", "attended_rows": pairs,
            "ms_bf16": round(ms_b, 5), "ms_q8_0": round(ms_q, 5), "speedup": round(ms_b / ms_q, 3),
            "bytes_bf16": by_b, "bytes_q8_0": by_q,
            "hbm_frac_bf16": by_b / (ms_b * 1e-3) / PEAK_HBM, "hbm_frac_q8_0": by_q / (ms_q * 1e-3) / PEAK_HBM,
            "mfma_frac_bf16": fl / (ms_b * 1e-3) / PEAK["bf16"], "mfma_frac_q8_0": fl / (ms_q * 1e-3) / PEAK["f16"],
            "linf_rel_q8_vs_bf16": round(linf, 5),
            "timing": "attention + split merge, caches flushed before each call" if flush is not None else "warm"}
        print(f"bench: q8_0 latent rows, {wl.name}: bf16 {ms_b:.4f} ms, q8_0 {ms_q:.4f} ms", file=sys.stderr,
              flush=True)
        del x, codes, scales, idx, out_b, out_q
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- main

def time_workload(dsa, inputs, torch, wl, steps, warmup, flush):
    """Times `steps` dsa_forward steps of workload wl (after `warmup` untimed
    ones), with the caches flushed before each timed step unless flush is
    None.  Returns (result dict, inputs)."""
    dev = "cuda"
    x = inputs.generate(wl, device=dev)
    kw = dict(k_scale=x["k_scale"], n_sink=wl.n_sink if wl.c == 1 else 0, scale=wl.scale,
              hadamard_q=wl.hadamard_q, kv_len=x["kv_len"])
    out = torch.empty((wl.S, wl.n_q, wl.Hq, wl.Dv), device=dev, dtype=torch.float32)
    nbytes = dsa.forward_workspace_bytes(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k,
                                         wl.c, x["q_pos"], **kw)
    ws = torch.empty(max(nbytes, 1), device=dev, dtype=torch.uint8)
    ev = [[dsa.Event() for _ in range(5)] for _ in range(steps)]
    ends = [[dsa.Event() for _ in range(2)] for _ in range(steps)]

    def step(events=None):
        dsa.forward(x["Q"], x["K"], x["V"], x["q_idx"], x["k_idx"], x["w"], wl.top_k, wl.c, x["q_pos"],
                    out=out, workspace=ws, phase_events=events, **kw)

    # warm-up steps in the timed loop's own pattern (the cache flush included):
    # steps without it leave the first ~10 flushed steps 5-30 % slower while
    # the GPU settles under the flush's 1 GiB reads
    for _ in range(warmup):
        if flush is not None:
            flush.amax()
        step()
    torch.cuda.synchronize()
    # The timed steps: the library records one event right before the step's
    # first launch and one after its last, nothing in between (the per-phase
    # events of the pass below cost about 2 us each on these short steps).
    # Events recorded by the caller around the call would also hold the
    # binding's argument marshalling, during which the GPU sits idle after
    # the cache flush (the host is slower than the GPU in this loop); that
    # figure is reported beside it (call_ms_per_step).
    t0 = time.perf_counter()
    for k in range(steps):
        if flush is not None:
            flush.amax()
        step([ends[k][0], None, None, None, ends[k][1]])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(ends[k][0].elapsed_ms(ends[k][1]) for k in range(steps))
    ms_step = sum(step_ms) / steps if flush is not None else elapsed * 1e3 / steps
    # the same steps bracketed by events around the call
    calls = [[dsa.Event() for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        if flush is not None:
            flush.amax()
        calls[k][0].record()
        step()
        calls[k][1].record()
    torch.cuda.synchronize()
    call_ms = sum(calls[k][0].elapsed_ms(calls[k][1]) for k in range(steps)) / steps
    # The same steps again with an event between the phases: the phase times
    # and the dominant kernel's launch time.
    for k in range(steps):
        if flush is not None:
            flush.amax()
        step(ev[k])
    torch.cuda.synchronize()
    phased_ms = sum(ev[k][0].elapsed_ms(ev[k][4]) for k in range(steps)) / steps
    warm_ms = None
    if flush is not None:   # the same steps back to back with warm caches, labelled as such
        n_warm = max(1, min(steps, 10))
        ew = [dsa.Event() for _ in range(2)]
        ew[0].record()
        for _ in range(n_warm):
            step()
        ew[1].record()
        torch.cuda.synchronize()
        warm_ms = ew[0].elapsed_ms(ew[1]) / n_warm

    # per-phase times from the HIP events recorded on the library's stream
    names = ["scores", "topk", "attn", "combine"]
    phase_ms = {n_: 0.0 for n_ in names}
    for k in range(steps):
        for j, n_ in enumerate(names):
            phase_ms[n_] += ev[k][j].elapsed_ms(ev[k][j + 1]) / steps

    work, pairs_score, pairs_attn = work_model(wl, x["q_pos"].cpu().numpy(), x["kv_len"].cpu().numpy())
    if wl.c > 1:   # pooling runs inside the first phase with the scores
        work["scores"] = {"flops": work["scores"]["flops"], "bytes": work["scores"]["bytes"] + work["pool"]["bytes"]}
    # the split merge runs in the attention phase's second launch: its time counts with attention
    phase_ms_attn = phase_ms["attn"] + phase_ms["combine"]
    cdt = compute_dtype(wl)
    per_phase = {}
    for n_ in ("scores", "topk", "attn"):
        t = max((phase_ms_attn if n_ == "attn" else phase_ms[n_]) * 1e-3, 1e-12)
        fl, by = work[n_]["flops"], work[n_]["bytes"]
        peak_f = PEAK["f16" if (n_ == "scores" and wl.k_dtype != torch.bfloat16 and cdt != "f32") else cdt]
        if n_ == "scores" and cdt == "f32":
            peak_f = PEAK["f32"]
        t_f, t_b = fl / peak_f, by / PEAK_HBM
        bound = "mfma" if t_f >= t_b else "hbm"
        if cdt == "f32" and bound == "mfma":
            bound = "alu"
        per_phase[n_] = dict(ms=t * 1e3, flops=fl, bytes=by, bound=bound,
                             frac=(t_f if bound != "hbm" else t_b) / t, peak=peak_f if bound != "hbm" else PEAK_HBM)
    # the dominant kernel: the longest single launch (attention without its merge)
    launch_ms = {"scores": phase_ms["scores"], "topk": phase_ms["topk"], "attn": phase_ms["attn"]}
    dom = max(launch_ms, key=lambda n_: launch_ms[n_])
    ph = per_phase[dom]
    t_dom = launch_ms[dom] * 1e-3
    if ph["bound"] in ("mfma", "alu"):
        roof = {"bound": ph["bound"], "achieved": ph["flops"] / t_dom / 1e12, "peak": ph["peak"] / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": ph["bytes"] / t_dom / 1e9, "peak": ph["peak"] / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = {"scores": score_kernel_name(wl), "topk": "topk kernels", "attn": attn_kernel_name(wl)}[dom]
    roof["traffic"] = measured_traffic(wl.name, roof["kernel"])
    roof["launch_ms"] = launch_ms[dom]
    step_bytes = sum(work[n_]["bytes"] for n_ in ("scores", "topk", "attn"))
    res = {
        "workload": wl.name,
        "query_tokens_per_s": wl.S * wl.n_q / (ms_step * 1e-3),
        "keys_scored_per_s": pairs_score / (ms_step * 1e-3),
        "keys_scored_per_s_score_phase": pairs_score / max(phase_ms["scores"] * 1e-3, 1e-12),
        "ms_per_step": ms_step,
        "config": {"workload": wl.name, "sequences": wl.S, "queries_per_sequence": wl.n_q, "cached_keys": wl.n_kv,
                   "indexer_heads": wl.H, "indexer_dim": wl.D, "indexer_key_dtype": str(wl.k_dtype).split(".")[1],
                   "top_k": wl.top_k, "compress_ratio": wl.c, "n_sink": wl.n_sink, "attention": wl.attn,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "dk": wl.Dk, "dv": wl.Dv,
                   "scored_pairs": pairs_score, "attended_pairs": pairs_attn},
        "dtype": cdt,
        "timing": {"cache": "flushed before each step (1 GiB read)" if flush is not None else "warm",
                   "steps": steps, "warmup": warmup,
                   "step_ms_median": round(step_ms[len(step_ms) // 2], 5),
                   "step_ms_p10": round(step_ms[int(0.1 * (len(step_ms) - 1))], 5),
                   "step_ms_p90": round(step_ms[int(0.9 * (len(step_ms) - 1))], 5),
                   "wall_ms_per_step": round(elapsed * 1e3 / steps, 5),
                   "ms_per_step_with_phase_events": round(phased_ms, 5),
                   "call_ms_per_step": round(call_ms, 5),
                   "warm_cache_ms_per_step": None if warm_ms is None else round(warm_ms, 5),
                   "step_clock": ("HIP events recorded by the library before the step's first launch and after "
                                  "its last" if flush is not None else "wall clock"),
                   "call_clock": "HIP events recorded by the caller around the dsa_forward call (its argument "
                                 "marshalling included)",
                   "phases_from": "a second pass of the same steps with an event between phases"},
        "phases_ms": {k_: round(v_, 5) for k_, v_ in phase_ms.items()},
        "phase_roofline": {k_: {"bound": v_["bound"], "frac": round(v_["frac"], 4)} for k_, v_ in per_phase.items()},
        # the whole step's algorithmic HBM bytes over its time (the decode workloads' bound)
        "step_hbm": {"bytes": step_bytes, "achieved_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac_of_8TBps": step_bytes / (ms_step * 1e-3) / PEAK_HBM},
        "roofline": roof,
    }
    return res, x


def calib_copy(torch):
    """One 1 GiB device-to-device copy: known bytes (1048576 KiB read and
    written) that calibrate the FETCH_SIZE / WRITE_SIZE counters of a run."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs on one GPU "
              "and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_top_attention_indexer_amd as dsa
    from sparse_top_attention_indexer_amd import inputs

    if args.next_rows_only:
        flush = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        print(json.dumps({"next_rows": {"index_key_write": key_write_row(dsa, inputs, torch, 20),
                                        "block_pool_update": pool_update_row(dsa, inputs, torch, 20),
                                        "index_share": index_share_row(dsa, inputs, torch, 5),
                                        "q8_0_latent": q8_latent_row(dsa, inputs, torch, 10, flush)}}),
              flush=True)
        if args.calib_copy:
            calib_copy(torch)
        return
    headline = args.config if args.config is not None else 2
    # Before each timed step a 1 GiB read evicts the L2s and the 256 MB
    # Infinity Cache, so that a step finds its inputs in HBM, as it would
    # after the other layers of a model ran.  A read leaves clean lines (a
    # write would leave dirty ones for the step to write back).  The flush
    # runs before the step's first library event, never inside the step.
    flush = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    wl = inputs.preset(headline)
    res, x = time_workload(dsa, inputs, torch, wl, args.steps, args.warmup, flush)
    line = {
        "metric": "query tokens/s + indexer keys scored/s (1 GPU), % of MFMA/HBM roofline",
        "value": res["query_tokens_per_s"],
        "unit": "query tokens/s",
        "keys_scored_per_s": res["keys_scored_per_s"],
        "keys_scored_per_s_score_phase": res["keys_scored_per_s_score_phase"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
        "data": "synthetic",
        "config": res["config"],
        "timing": res["timing"],
        "phases_ms": res["phases_ms"],
        "phase_roofline": res["phase_roofline"],
        "step_hbm": res["step_hbm"],
        "roofline": res["roofline"],
    }
    print(f"bench: workload {wl.name} done, {res['ms_per_step']:.4f} ms per step", file=sys.stderr, flush=True)
    if args.config is None and not args.headline_only:
        # the other workloads, same protocol, fewer steps; inputs freed in turn
        others = {}
        for n in (1, 3, 4, 5):
            wl_n = inputs.preset(n)
            r, xn = time_workload(dsa, inputs, torch, wl_n, min(args.steps, 10), args.warmup, flush)
            del xn
            torch.cuda.empty_cache()
            others[wl_n.name] = {k_: r[k_] for k_ in ("query_tokens_per_s", "keys_scored_per_s",
                                                       "keys_scored_per_s_score_phase", "ms_per_step", "dtype",
                                                       "timing", "phases_ms", "phase_roofline", "step_hbm",
                                                       "roofline")}
            print(f"bench: workload {wl_n.name} done, {r['ms_per_step']:.4f} ms per step", file=sys.stderr,
                  flush=True)
        line["configs"] = others
    if not args.no_next_rows:
        line["next_rows"] = {"index_key_write": key_write_row(dsa, inputs, torch, 20),
                             "block_pool_update": pool_update_row(dsa, inputs, torch, 20),
                             "index_share": index_share_row(dsa, inputs, torch, 5),
                             "q8_0_latent": q8_latent_row(dsa, inputs, torch, 10, flush)}
    if args.calib_copy:
        calib_copy(torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds)
        if headline in (1, 3):   # the small and the batched-decode workloads also on one core
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                one = cpu_baseline(wl, x, args.cpu_seconds / 2)
            line["cpu_baseline"]["one_core"] = {k: one[k] for k in ("value", "keys_scored_per_s", "sample")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
