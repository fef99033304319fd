#!/usr/bin/env python3
"""Throughput of the TurboQuant compressed-KV hot path on one MI355X.

One step = quantize-on-append of the new tokens of every (batch, KV head)
for K (token-major records) and V (32-token block records), then one decode
step over the whole compressed cache: tq_attn_decode_append, i.e. one launch
for both appends and the query prep, then the split-K pass and the combine.
The default workload is the 70B-shaped long context (batch 4, 64 query / 8
KV heads, 131072 tokens, 3 bits): an 8192-token chunk is quantized per head
(524,288 vectors), then one decode step attends over all 131072 tokens.
Inputs are seeded synthetic tensors already resident in HBM; the cache is
built (untimed) by the library's own quantize kernel from synthetic K/V.

To measure HBM rather than the 256 MB Infinity Cache, each step uses the
next of several copies of the compressed cache (at least 1 GiB in total).

Prints one JSON line: cached tokens/s (batch * context / step time), the
split-K kernel against the HBM roofline (HIP events around that kernel on
its stream), the same decode for the other decode workloads, quantize
throughput, the decode over uncompressed bf16 K/V for comparison, the
nearest-neighbour search workload, and the CPU oracle timed on a bounded
sample as a baseline.
"""
from __future__ import annotations

import os
import sys


def _host_cores() -> int:
    """Host threads the oracle may use: the process's CPU affinity, capped by
    OMP_NUM_THREADS when the environment sets it."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    lim = os.environ.get("OMP_NUM_THREADS", "")
    if lim.isdigit() and int(lim) > 0:
        n = min(n, int(lim))
    return max(1, n)


# BLAS and OpenMP pools size themselves when numpy is first imported, so the
# thread count is fixed here, before any import that loads numpy.
HOST_CORES = _host_cores()
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
    os.environ[_var] = str(HOST_CORES)

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import math  # noqa: E402
import time  # noqa: E402
from concurrent.futures import ThreadPoolExecutor  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix, vendor figure
PEAK_FP16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix, vendor figure
DECODE_WORKLOADS = ("llama8b_decode", "llama70b_long", "mixed_3p5", "mixed_2p5")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_traffic.json")
DECODE_SOURCE = os.path.join(ROOT, "kv_cache_vector_rotation_amd", "csrc", "tq_decode.hip")
COPY_PROBE_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_long", choices=DECODE_WORKLOADS)
    ap.add_argument("--copies", type=int, default=0, help="cache copies (0: enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize-bench", action="store_true")
    ap.add_argument("--no-decode-legs", action="store_true",
                    help="skip the other decode workloads (llama8b_decode, mixed_3p5, mixed_2p5)")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true")
    ap.add_argument("--no-chunk", action="store_true", help="skip the prefill-chunk and paged-cache legs")
    ap.add_argument("--no-mixed", action="store_true", help="(same as --no-decode-legs)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the record-variant legs (MSE-only V, fp16 norms)")
    ap.add_argument("--ctx-sweep", default="",
                    help="comma-separated context lengths: also time the compressed step and the bf16 "
                         "decode of the llama8b_decode shape at each (reported under ctx_sweep)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (the reference for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return ap.parse_args()


def record_bytes(dims, bits):
    return sum((m + 1) * d for d, m in zip(dims, bits)) / 8 + 8 * len(dims)


def _threads():
    """Worker threads for drawing synthetic slabs on the host."""
    return max(1, min(16, HOST_CORES))


def build_caches(tq, torch, wl, kq, vq, prefix, cap, device_fill=False):
    """Quantize tokens [0, prefix) of every (b, h) into fresh caches (untimed);
    device_fill: the tokens are N(0, 1) bf16 vectors drawn on the device (for
    large batches, where drawing the synthetic slabs on the host is slow)."""
    B, H = wl.batch, wl.n_kv_heads
    kc = tq.Cache.empty(kq, B * H * cap, tq.TQ_TOKEN_MAJOR)
    vc = tq.Cache.empty(vq, B * H * cap, tq.TQ_BLOCK32)
    if prefix == 0:
        return kc, vc
    if device_fill:
        g = torch.Generator(device="cuda")
        g.manual_seed(wl.seed)
        for b in range(B):
            for qz, cache, fmt in ((kq, kc, tq.TQ_TOKEN_MAJOR), (vq, vc, tq.TQ_BLOCK32)):
                x = torch.randn((H * prefix, wl.d), generator=g, device="cuda").to(torch.bfloat16)
                tq.tq_quantize(qz, fmt, x, cache, seg_len=prefix, seg_stride=cap, seg_offset=b * H * cap)
        torch.cuda.synchronize()
        return kc, vc
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    pairs = [(b, h) for b in range(B) for h in range(H)]
    per = max(1, min(len(pairs), int(2e9 // (prefix * wl.d * 8))))
    with ThreadPoolExecutor(_threads()) as ex:
        for i in range(0, len(pairs), per):
            chunk = pairs[i:i + per]
            ks = list(ex.map(lambda p: synth.draw_kv_slab(wl, "K", p[0], p[1], 0, prefix), chunk))
            vs = list(ex.map(lambda p: synth.draw_kv_slab(wl, "V", p[0], p[1], 0, prefix), chunk))
            for (b, h), kx, vx in zip(chunk, ks, vs):
                row0 = (b * H + h) * cap
                for x, qz, cache, fmt in ((kx, kq, kc, tq.TQ_TOKEN_MAJOR), (vx, vq, vc, tq.TQ_BLOCK32)):
                    xt = torch.from_numpy(x).cuda().to(dt)
                    tq.tq_quantize(qz, fmt, xt, cache, seg_len=prefix, seg_stride=cap, seg_offset=row0)
            torch.cuda.synchronize()
    return kc, vc


def new_tokens(torch, wl, prefix):
    B, H = wl.batch, wl.n_kv_heads
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    pairs = [(b, h) for b in range(B) for h in range(H)]
    with ThreadPoolExecutor(_threads()) as ex:
        ks = list(ex.map(lambda p: synth.draw_kv_slab(wl, "K", p[0], p[1], prefix, wl.n_ctx), pairs))
        vs = list(ex.map(lambda p: synth.draw_kv_slab(wl, "V", p[0], p[1], prefix, wl.n_ctx), pairs))
    k = torch.from_numpy(np.concatenate(ks)).cuda().to(dt)
    v = torch.from_numpy(np.concatenate(vs)).cuda().to(dt)
    return k, v


def traffic_record(workload):
    """HBM bytes per launch of the split-K kernel on ``workload`` from
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters, if they were taken on the
    current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    sha = hashlib.sha256(open(DECODE_SOURCE, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha or workload not in rec.get("workloads", {}):
        return None
    return dict(rec["workloads"][workload], kernel=rec.get("kernel"))


def _quantize_timed(tq, torch, calls, launches):
    """Mean seconds per round of ``calls`` (quantize launches), HIP events."""
    for _ in range(3):
        for c in calls:
            c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        for c in calls:
            c()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / launches


def quantize_chunk_bench(tq, torch, launches=20):
    """The prefill-chunk quantize of the llama70b_long step on its own: the
    8192-token chunk of every (batch, KV head), K into token-major records
    and V into 32-token block records at the step's rows (524,288 vectors,
    3 bits), as two tq_quantize launches."""
    wl = synth.workload("llama70b_long")
    ks, vs = synth.draw_quantizer(wl, "K"), synth.draw_quantizer(wl, "V")
    bits = [g.mse_bits for g in ks.groups]
    kq = tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm)
    vq = tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm)
    B, H, cap = wl.batch, wl.n_kv_heads, wl.capacity
    prefix = wl.n_ctx - wl.n_new
    k_new, v_new = new_tokens(torch, wl, prefix)
    kc = tq.Cache.empty(kq, B * H * cap, tq.TQ_TOKEN_MAJOR)
    vc = tq.Cache.empty(vq, B * H * cap, tq.TQ_BLOCK32)
    kw = dict(seg_len=wl.n_new, seg_stride=cap, seg_offset=prefix)
    calls = [lambda: tq.tq_quantize(kq, tq.TQ_TOKEN_MAJOR, k_new, kc, **kw),
             lambda: tq.tq_quantize(vq, tq.TQ_BLOCK32, v_new, vc, **kw)]
    s = _quantize_timed(tq, torch, calls, launches)
    n_vec = 2 * B * H * wl.n_new
    # bf16 rows, d <= 128: the rotation runs as three bf16 products and the
    # sketch product as three fp16 products (two-part operands), so the
    # matrix cores issue 6 x 2 d^2 flops per vector against the 16-bit peak;
    # HBM moves the bf16 row in and the record out
    issued = 6 * 2.0 * wl.d * wl.d * n_vec
    hbm = n_vec * (2 * wl.d + record_bytes([wl.d], bits))
    del kc, vc, k_new, v_new
    return {"workload": "llama70b_long", "vectors": n_vec, "formats": "K token-major + V block32",
            "bits_per_channel": [m + 1 for m in bits], "input_dtype": wl.dtype,
            "us_per_chunk": round(s * 1e6, 2), "vectors_per_s": n_vec / s,
            "mfma_products": "rotation 3 x bf16, sketch 3 x fp16 (fp32 accumulation)",
            "mfma_issued_tflops": round(issued / s / 1e12, 1), "mfma_peak_tflops": PEAK_FP16_MFMA_TFLOPS,
            "mfma_frac": round(issued / s / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4),
            "hbm_gbs": round(hbm / s / 1e9, 1), "hbm_frac": round(hbm / s / 1e9 / PEAK_HBM_GBS, 4),
            "bound": "VALU issue and latency (neither matrix cores nor HBM are near their peaks)"}


def quantize_nn_bench(tq, torch, launches=5):
    """The nearest-neighbour database quantize: 1,000,000 fp32 vectors of
    d = 200 at 4 bits (3 + 1) into token-major records, one launch."""
    wl = synth.workload("nn_search")
    spec = synth.draw_quantizer(wl, "K")
    qz = tq.Quantizer.from_parts(spec.rotations, spec.sketches, [g.mse_bits for g in spec.groups], perm=spec.perm)
    x = torch.from_numpy(synth.draw_mixture_vectors(wl, wl.n_ctx, "db")).cuda()
    db = tq.Cache.empty(qz, wl.n_ctx, tq.TQ_TOKEN_MAJOR)
    calls = [lambda: tq.tq_quantize(qz, tq.TQ_TOKEN_MAJOR, x, db, seg_len=wl.n_ctx, seg_stride=wl.n_ctx)]
    s = _quantize_timed(tq, torch, calls, launches)
    flops = 4.0 * wl.d * wl.d * wl.n_ctx
    del x, db
    return {"workload": "nn_search", "vectors": wl.n_ctx, "d": wl.d, "bits_per_channel": 4, "input_dtype": "f32",
            "us_per_launch": round(s * 1e6, 2), "vectors_per_s": wl.n_ctx / s,
            "bound": "mfma", "achieved_tflops": round(flops / s / 1e12, 2), "peak_tflops": PEAK_FP32_MFMA_TFLOPS,
            "peak_kind": "fp32 MFMA", "frac": round(flops / s / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4)}


def bf16_baseline(tq, torch, wl, q, step_ms, launches=200, min_bytes=1 << 30, max_copies=None):
    """Secondary figure: the same decode over uncompressed bf16 K/V caches
    (tq_attn_decode_bf16: split-K pass and combine), on copies of the cache
    totalling at least 1 GiB so that it streams from HBM. Returns its time
    per decode, its bandwidth against the HBM roofline and the ratio to the
    compressed step time (which also includes the appends)."""
    B, HQ, H, d, N = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.d, wl.n_ctx
    cap = wl.capacity
    pairs = [(b, h) for b in range(B) for h in range(H)]
    k = torch.empty((B * H * cap, d), dtype=torch.bfloat16, device="cuda")
    vt = torch.empty((B * H * cap, d), dtype=torch.bfloat16, device="cuda")
    per = max(1, min(len(pairs), int(2e9 // (N * d * 8))))
    with ThreadPoolExecutor(_threads()) as ex:
        for i in range(0, len(pairs), per):
            chunk = pairs[i:i + per]
            ks = list(ex.map(lambda p: synth.draw_kv_slab(wl, "K", p[0], p[1], 0, N), chunk))
            vs = list(ex.map(lambda p: synth.draw_kv_slab(wl, "V", p[0], p[1], 0, N), chunk))
            for (b, h), kx, vx in zip(chunk, ks, vs):
                r0 = (b * H + h) * cap
                k[r0:r0 + N] = torch.from_numpy(kx).cuda().to(torch.bfloat16)
                vt[r0:r0 + N] = torch.from_numpy(vx).cuda().to(torch.bfloat16)
    v = vt.reshape(B * H * cap // 32, 32, d).transpose(1, 2).contiguous()
    del vt
    cache_bytes = 2 * k.numel() * 2
    n_copies = max(1, math.ceil(min_bytes / cache_bytes))
    if max_copies:
        n_copies = min(n_copies, max_copies)
    caches = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n_copies - 1)]
    shape = tq.decode_shape(B, HQ, H, N, cap, wl.scale)
    ws = torch.empty(tq.tq_attn_decode_bf16_workspace_bytes(shape, d), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, HQ, d), dtype=torch.float32, device="cuda")
    for i in range(n_copies):
        tq.tq_attn_decode_bf16(shape, q, caches[i][0], caches[i][1], out, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_copies):
            tq.tq_attn_decode_bf16(shape, q, caches[i][0], caches[i][1], out, workspace=ws)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(launches / n_copies))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_copies)
    algo = B * H * N * d * 2 * 2  # bf16 K and V of every cached token
    gbs = algo / (ms / 1e3) / 1e9
    del caches, k, v
    return {"kernel": "bf16_split_kernel + bf16_combine_kernel", "us_per_decode": round(ms * 1e3, 2),
            "cached_tokens_per_s": B * N / (ms / 1e3), "algorithmic_bytes": int(algo),
            "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "cache_copies": n_copies, "compressed_step_speedup": round(ms / step_ms, 3)}




def search_bench(tq, torch, reps=5):
    """Secondary figure: nearest-neighbour search on the nn_search workload
    (1,000,000 database vectors, d = 200, 4 bits; 10,000 queries; top 10):
    the database is quantized on the device, then tq_search is timed with HIP
    events. Reports queries/s, the dense-equivalent fp16 TFLOP/s of the scan
    (2 flop x n_q x n_db x d for each of the rotated and the sketch products)
    against the dense fp16 MFMA peak, and recall@10 against exact fp32 brute
    force (torch matmul and top-k, query chunks)."""
    wl = synth.workload("nn_search")
    n_db, n_q, k = wl.n_ctx, 10_000, 10
    spec = synth.draw_quantizer(wl, "K")
    qz = tq.Quantizer.from_parts(spec.rotations, spec.sketches, [g.mse_bits for g in spec.groups], perm=spec.perm)
    x = torch.from_numpy(synth.draw_mixture_vectors(wl, n_db, "db")).cuda()
    q = torch.from_numpy(synth.draw_mixture_vectors(wl, n_q, "query")).cuda()
    db = tq.Cache.empty(qz, n_db, tq.TQ_TOKEN_MAJOR)
    tq.tq_quantize(qz, tq.TQ_TOKEN_MAJOR, x, db, seg_len=n_db, seg_stride=n_db)
    ws = torch.empty(tq.tq_search_workspace_bytes(qz, n_db, n_q, k), dtype=torch.uint8, device="cuda")
    oi = torch.empty((n_q, k), dtype=torch.int64, device="cuda")
    osc = torch.empty((n_q, k), dtype=torch.float32, device="cuda")
    tq.tq_search(qz, db, n_db, q, k, out_idx=oi, out_score=osc, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tq.tq_search(qz, db, n_db, q, k, out_idx=oi, out_score=osc, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    hits = 0
    for s0 in range(0, n_q, 1000):
        ex = torch.topk(q[s0:s0 + 1000] @ x.T, k, dim=1).indices
        got = oi[s0:s0 + 1000]
        hits += int((got[:, :, None] == ex[:, None, :]).any(dim=2).sum())
    flop = 2.0 * 2 * n_q * n_db * wl.d
    tf = flop / (ms / 1e3) / 1e12
    del x, db, ws
    return {"workload": "nn_search", "n_db": n_db, "n_q": n_q, "d": wl.d, "k": k, "bits_per_channel": 4,
            "ms_per_search": round(ms, 3), "queries_per_s": n_q / (ms / 1e3),
            "bound": "mfma", "dense_equiv_tflops": round(tf, 1), "peak_tflops": PEAK_FP16_MFMA_TFLOPS,
            "frac": round(tf / PEAK_FP16_MFMA_TFLOPS, 4), "recall_at_10": hits / (n_q * k)}


def compressed_step_us(tq, torch, wl, kq, vq, n_copies, reps=20, T=1, device_fill=False):
    """Mean time of tq_attn_decode_append steps (graph of one step per cache
    copy, replayed), in microseconds. T > 1: a causal chunk of T query tokens
    per head (the workload's last T tokens are the ones appended)."""
    B, HQ, H, N, cap = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_ctx, wl.capacity
    prefix = N - wl.n_new
    kc0, vc0 = build_caches(tq, torch, wl, kq, vq, prefix, cap, device_fill)
    caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(n_copies - 1)]
    k_new, v_new = new_tokens(torch, wl, prefix)
    if T == 1:
        qn = synth.draw_queries(wl)
    else:
        qn = synth.to_bf16_exact(synth.standard_normal(synth.rng_for(wl.seed, 21, T), (B, T, HQ, wl.d)))
    q = torch.from_numpy(qn).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, HQ, H, N, cap, wl.scale, n_q_tokens=T)
    ws = torch.empty(tq.tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, T, HQ, wl.d), dtype=torch.float32, device="cuda")
    k_app = tq.append_spec(k_new, seg_len=wl.n_new, seg_stride=cap, seg_offset=prefix)
    v_app = tq.append_spec(v_new, seg_len=wl.n_new, seg_stride=cap, seg_offset=prefix)

    def step(i):
        tq.tq_attn_decode_append(kq, vq, shape, q, caches[i][0], caches[i][1], k_new=k_app, v_new=v_app,
                                 out=out, workspace=ws)
    for i in range(n_copies):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_copies):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_copies)


def _llama8b_quantizers(tq):
    base = synth.workload("llama8b_decode")
    ks, vs = synth.draw_quantizer(base, "K"), synth.draw_quantizer(base, "V")
    bits = [g.mse_bits for g in ks.groups]
    return (tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm),
            tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm))


def variants_bench(tq, torch):
    """Secondary figures: the llama8b_decode step (append + decode) with the
    record variants: MSE-only V records (stage one alone: the same code bits,
    no sign bits) under two-stage K; fp16 norms in both caches; both. Each
    over enough cache copies for 1 GiB."""
    wl = synth.workload("llama8b_decode")
    ks, vs = synth.draw_quantizer(wl, "K"), synth.draw_quantizer(wl, "V")
    bits = [g.mse_bits for g in ks.groups]
    dims = [g.dim for g in ks.groups]
    out = {"workload": "llama8b_decode"}
    for name, v_mse, f16 in (("mse_only_v", True, False), ("fp16_norms", False, True),
                             ("mse_only_v_fp16_norms", True, True)):
        kq = tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm, norm_f16=f16)
        vq = tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm, mse_only=v_mse,
                                     norm_f16=f16)
        nb = (4 if f16 else 8) * len(dims)
        rb_k = sum((m + 1) * d for d, m in zip(dims, bits)) / 8 + nb
        rb_v = sum((m if v_mse else m + 1) * d for d, m in zip(dims, bits)) / 8 + nb
        copies = max(1, math.ceil((1 << 30) / (wl.batch * wl.n_kv_heads * wl.capacity * (rb_k + rb_v))))
        us = compressed_step_us(tq, torch, wl, kq, vq, copies)
        out[name] = {"us_per_step": round(us, 2), "cached_tokens_per_s": wl.batch * wl.n_ctx / (us / 1e6),
                     "record_bytes_per_token": {"K": rb_k, "V": rb_v}, "cache_copies": copies}
    return out


def decode_leg(tq, torch, wl, steps, warmup=3, copies=0, device_fill=False, split_launches=200):
    """The fused step (appends + decode) of workload ``wl`` and its split-K
    kernel alone. Every step uses the next of several cache copies (at least
    1 GiB in total). Exactly ``steps`` steps are timed: one HIP graph holds a
    cycle of one step per copy and is replayed steps // copies times, and a
    second graph holds the remaining steps % copies steps. The split-K pass is
    timed alone from replays of a graph of split-K launches, one per copy,
    between HIP events on the launch stream."""
    B, HQ, H, d, N = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.d, wl.n_ctx
    cap = wl.capacity
    prefix = N - wl.n_new
    ks, vs = synth.draw_quantizer(wl, "K"), synth.draw_quantizer(wl, "V")
    bits = [g.mse_bits for g in ks.groups]
    dims = [g.dim for g in ks.groups]
    kq = tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm)
    vq = tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm)
    t0 = time.perf_counter()
    kc0, vc0 = build_caches(tq, torch, wl, kq, vq, prefix, cap, device_fill)
    k_new, v_new = new_tokens(torch, wl, prefix)
    rb = record_bytes(dims, bits)
    cache_bytes = B * H * cap * 2 * rb
    n_copies = copies or max(1, math.ceil((1 << 30) / cache_bytes))
    caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(n_copies - 1)]
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(dt)
    shape = tq.decode_shape(B, HQ, H, N, cap, wl.scale)
    ws = torch.empty(tq.tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, HQ, d), dtype=torch.float32, device="cuda")
    k_app = tq.append_spec(k_new, seg_len=wl.n_new, seg_stride=cap, seg_offset=prefix)
    v_app = tq.append_spec(v_new, seg_len=wl.n_new, seg_stride=cap, seg_offset=prefix)
    torch.cuda.synchronize()
    log(f"{wl.name}: setup {time.perf_counter() - t0:.1f}s B={B} Hq={HQ} Hkv={H} d={d} N={N} bits={bits} "
        f"dims={dims} copies={n_copies} ({n_copies * cache_bytes / 2**30:.2f} GiB)")

    def step(i):
        kc, vc = caches[i % n_copies]
        tq.tq_attn_decode_append(kq, vq, shape, q, kc, vc, k_new=k_app, v_new=v_app, out=out, workspace=ws)

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    full, rem = divmod(steps, n_copies)
    g_full = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_full):
        for i in range(n_copies):
            step(i)
    g_rem = None
    if rem:
        g_rem = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rem):
            for i in range(rem):
                step(i)
    g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / steps
    # the split-K pass alone (the prepared queries in the workspace are the
    # same for every copy)
    g_split = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_split):
        for i in range(n_copies):
            kc, vc = caches[i]
            tq.tq_attn_decode_phases(tq.TQ_PHASE_SPLIT, kq, vq, shape, q, kc, vc, out=out, workspace=ws)
    g_split.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(split_launches / n_copies))
    split_ms = []
    for _ in range(5):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            g_split.replay()
        a1.record()
        torch.cuda.synchronize()
        split_ms.append(a0.elapsed_time(a1) / (reps * n_copies))
    split_s = float(np.mean(split_ms)) / 1e3
    algo = B * H * N * 2 * rb  # every K and V record read once by the split-K pass
    gbs = algo / split_s / 1e9
    log(f"{wl.name}: step {ms_step * 1e3:.2f} us over {steps} steps (wall {wall / steps * 1e6:.2f} us); split-K "
        f"mean {split_s * 1e6:.2f} us (median {np.median(split_ms) * 1e3:.2f}, min {np.min(split_ms) * 1e3:.2f}) "
        f"-> {gbs:.0f} GB/s, {gbs / PEAK_HBM_GBS:.3f} of peak")
    res = {"workload": wl.name, "steps": steps, "us_per_step": round(ms_step * 1e3, 3),
           "cached_tokens_per_s": B * N / (ms_step / 1e3), "record_bytes_per_token": rb,
           "cache_copies": n_copies, "split_kernel_us": round(split_s * 1e6, 3),
           "split_algorithmic_bytes": int(algo), "split_achieved_gbs": round(gbs, 1),
           "split_frac": round(gbs / PEAK_HBM_GBS, 4),
           "step_frac_of_hbm_peak": round(algo / (ms_step / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
    if device_fill:
        res["cache_fill"] = "device-drawn N(0,1) bf16 tokens"
    state = dict(q=q, ms_step=ms_step, kq=kq, vq=vq)
    del caches, kc0, vc0, g_full, g_rem, g_split, ws
    torch.cuda.empty_cache()
    return res, state


def decode_legs(tq, torch, names):
    """Secondary decode workloads: each one's fused step and split-K kernel."""
    out = {}
    for name in names:
        wl = synth.workload(name)
        fill = wl.batch * wl.n_kv_heads * wl.n_ctx > 8 * 32768  # large caches: device-drawn tokens
        steps = 40 if fill else 290
        out[name], _ = decode_leg(tq, torch, wl, steps, device_fill=fill)
    return out


def chunk_bench(tq, torch, T=64):
    """Secondary figure: a prefill chunk on the llama8b_decode shape: T new
    tokens per KV head appended (K and V) and T x 32 query tokens attended
    causally over the 32768-token cache, one tq_attn_decode_append call."""
    wl = synth.workload("llama8b_decode", n_new=T)
    kq, vq = _llama8b_quantizers(tq)
    rb = record_bytes([g for g, _ in wl.groups], [m for _, m in wl.groups])
    copies = max(1, math.ceil((1 << 30) / (wl.batch * wl.n_kv_heads * wl.capacity * 2 * rb)))
    us = compressed_step_us(tq, torch, wl, kq, vq, copies, T=T)
    # the split-K pass decodes each 32-token tile once per workgroup and runs
    # 16-column blocks of the G T columns of a KV head on it: per (tile,
    # block) three K products (q_rot hi, q_rot lo, q_sk) of 32 x 128 x 16 and
    # two V products (codes, signs) of 128 x 32 x 16
    cache_bytes = wl.batch * wl.n_kv_heads * wl.n_ctx * 2 * rb
    cols = wl.n_q_heads // wl.n_kv_heads * T
    flop = wl.batch * wl.n_kv_heads * (wl.n_ctx // 32) * (cols // 16) * 2 * 16 * 32 * wl.d * (3 + 2)
    return {"workload": "llama8b_decode", "query_tokens_per_head": T, "n_ctx": wl.n_ctx,
            "us_per_chunk": round(us, 2), "query_tokens_per_s": wl.batch * T / (us / 1e6),
            "cache_copies": copies, "split_kernel": "chunk_kernel (each tile decoded once per workgroup)",
            "cache_bytes_read": cache_bytes, "hbm_gbs": round(cache_bytes / us / 1e3, 1),
            "hbm_frac": round(cache_bytes / us / 1e3 / PEAK_HBM_GBS, 4),
            "mfma_issued_tflops": round(flop / us / 1e6, 1), "mfma_peak_tflops": PEAK_FP16_MFMA_TFLOPS,
            "mfma_frac": round(flop / us / 1e6 / PEAK_FP16_MFMA_TFLOPS, 4),
            "bound": "per-column logit, softmax and V work with two waves per SIMD (neither HBM nor the "
                     "matrix cores near their peaks); times are of the whole chunk step"}


def paged_bench(tq, torch, n_copies=8, reps=20):
    """Secondary figure: the llama8b_decode decode (prep, split-K, combine; no
    append) through tq_attn_decode_paged with a shuffled block table, against
    tq_attn_decode on the contiguous cache holding the same records; both
    over n_copies rotated cache copies."""
    wl = synth.workload("llama8b_decode")
    kq, vq = _llama8b_quantizers(tq)
    B, HQ, H, N, cap = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_ctx, wl.capacity
    kc0, vc0 = build_caches(tq, torch, wl, kq, vq, N, cap)
    mb = cap // 32
    perm = torch.from_numpy(np.random.default_rng(7).permutation(B * mb).astype(np.int64)).cuda()
    table = perm.view(B, mb).to(torch.int32).contiguous()
    # physical block p holds logical block j of batch b where perm[b mb + j] = p
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(B * mb, device="cuda")
    info = tq.tq_record_layout(kq.layout)
    b_of = inv // mb
    j_of = inv % mb
    hh = torch.arange(H, device="cuda")
    src_blk = ((b_of[:, None] * H + hh[None, :]) * mb + j_of[:, None]).reshape(-1)  # contiguous 32-row block
    src_rows = (src_blk[:, None] * 32 + torch.arange(32, device="cuda")[None, :]).reshape(-1)
    kp = tq.Cache(fmt=tq.TQ_TOKEN_MAJOR, n_rows=kc0.n_rows,
                  codes=kc0.codes.view(-1, info.code_words)[src_rows].reshape(-1).contiguous(),
                  signs=kc0.signs.view(-1, info.sign_words)[src_rows].reshape(-1).contiguous(),
                  norms=kc0.norms.view(-1, info.norm_floats)[src_rows].reshape(-1).contiguous())
    vp = tq.Cache(fmt=tq.TQ_BLOCK32, n_rows=vc0.n_rows,
                  codes=vc0.codes.view(-1, info.block_code_words)[src_blk].reshape(-1).contiguous(),
                  signs=vc0.signs.view(-1, info.block_sign_words)[src_blk].reshape(-1).contiguous(),
                  norms=vc0.norms.view(-1, info.norm_floats)[src_rows].reshape(-1).contiguous())
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, HQ, H, N, cap, wl.scale)
    ws = torch.empty(tq.tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, HQ, wl.d), dtype=torch.float32, device="cuda")
    res = {}
    for name, pair in (("contiguous", (kc0, vc0)), ("paged", (kp, vp))):
        copies = [pair] + [(pair[0].clone(), pair[1].clone()) for _ in range(n_copies - 1)]

        def call(i):
            k, v = copies[i]
            if name == "paged":
                tq.tq_attn_decode_paged(kq, vq, shape, table, q, k, v, out=out, workspace=ws)
            else:
                tq.tq_attn_decode(kq, vq, shape, q, k, v, out=out, workspace=ws)
        for i in range(n_copies):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_copies):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / (reps * n_copies)
        del copies
    return {"workload": "llama8b_decode", "us_per_decode_contiguous": round(res["contiguous"], 2),
            "us_per_decode_paged": round(res["paged"], 2), "cache_copies": n_copies,
            "block_table": "shuffled 32-token blocks"}


def ctx_sweep(tq, torch, contexts):
    """Compressed step against the bf16 baseline decode at several context
    lengths of the llama8b_decode shape (both over rotated cache copies of at
    least 256 MiB, at most 64 copies)."""
    rows = []
    base = synth.workload("llama8b_decode")
    ks, vs = synth.draw_quantizer(base, "K"), synth.draw_quantizer(base, "V")
    bits = [g.mse_bits for g in ks.groups]
    kq = tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm)
    vq = tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm)
    for n in contexts:
        wl = synth.workload("llama8b_decode", n_ctx=n)
        rb = record_bytes([g for g, _ in wl.groups], [m for _, m in wl.groups])
        comp_bytes = wl.batch * wl.n_kv_heads * wl.capacity * 2 * rb
        copies = max(1, min(64, math.ceil((256 << 20) / comp_bytes)))
        step_us = compressed_step_us(tq, torch, wl, kq, vq, copies)
        q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
        b = bf16_baseline(tq, torch, wl, q, step_us / 1e3, min_bytes=256 << 20, max_copies=64)
        rows.append({"n_ctx": n, "compressed_step_us": round(step_us, 2), "compressed_copies": copies,
                     "bf16_decode_us": b["us_per_decode"], "bf16_copies": b["cache_copies"],
                     "compressed_step_speedup": b["compressed_step_speedup"]})
        log(f"ctx {n}: compressed step {step_us:.2f} us, bf16 decode {b['us_per_decode']:.2f} us")
        torch.cuda.empty_cache()
    return rows


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return HOST_CORES


def cpu_baseline(wl, budget_s):
    """The oracle (plain float64 numpy) on a bounded sample of the same step:
    for (b, h) pairs in order, untimed: quantize the prefix; timed: quantize
    the appended token(s), dequantize the K and V caches and attend with the
    pair's query heads. The mean time per pair is scaled to the whole step.
    Also the tiny workload's oracle (quantize 4096 keys, 64 x 4096 logits)
    with all host threads and with one thread."""
    import oracle  # the baseline leg is the only bench code that uses the oracle
    okq = oracle.Quantizer.from_spec(synth.draw_quantizer(wl, "K"))
    ovq = oracle.Quantizer.from_spec(synth.draw_quantizer(wl, "V"))
    q = synth.draw_queries(wl).astype(np.float64)
    G = wl.group_size
    prefix = wl.n_ctx - wl.n_new
    times, pairs_done, started = [], 0, time.perf_counter()
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            kx = synth.draw_kv_slab(wl, "K", b, h, 0, wl.n_ctx)
            vx = synth.draw_kv_slab(wl, "V", b, h, 0, wl.n_ctx)
            kp, vp = oracle.quantize(kx[:prefix], okq), oracle.quantize(vx[:prefix], ovq)
            t0 = time.perf_counter()
            kn, vn = oracle.quantize(kx[prefix:], okq), oracle.quantize(vx[prefix:], ovq)
            cat = lambda a, c: [np.concatenate([u, w]) for u, w in zip(a, c)]
            kt = oracle.dequantize(cat(kp.idx, kn.idx), cat(kp.bits, kn.bits), cat(kp.norm, kn.norm),
                                   cat(kp.gamma, kn.gamma), okq)
            vt = oracle.dequantize(cat(vp.idx, vn.idx), cat(vp.bits, vn.bits), cat(vp.norm, vn.norm),
                                   cat(vp.gamma, vn.gamma), ovq)
            oracle.attention_decode(q[b, h * G:(h + 1) * G], kt[None], vt[None], wl.scale)
            times.append(time.perf_counter() - t0)
            pairs_done += 1
            if sum(times) >= budget_s or time.perf_counter() - started > 4 * budget_s:
                break
        else:
            continue
        break
    per_step = float(np.mean(times)) * wl.batch * wl.n_kv_heads
    # the tiny workload with every host thread and with one
    tiny = synth.workload("tiny")
    tspec = synth.draw_quantizer(tiny, "K")
    tq_o = oracle.Quantizer.from_spec(tspec)
    tk = synth.draw_kv_slab(tiny, "K", 0, 0, 0, tiny.n_ctx)
    tqr = synth.draw_queries(tiny)[0].astype(np.float64)

    def tiny_run():
        t0 = time.perf_counter()
        qv = oracle.quantize(tk, tq_o)
        kt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, tq_o)
        oracle.estimate_logits(tqr, kt, tiny.scale)
        return time.perf_counter() - t0
    tiny_all = min(tiny_run() for _ in range(3))
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            tiny_one = min(tiny_run() for _ in range(3))
    except Exception:  # pragma: no cover
        tiny_one = None
    return {"value": wl.batch * wl.n_ctx / per_step, "unit": "cached tokens/s", "cores": int(_blas_threads()),
            "kind": "oracle",
            "sample": f"{pairs_done} of {wl.batch * wl.n_kv_heads} (batch, KV head) pairs of {wl.name}: append "
                      f"{wl.n_new} token(s) K+V, dequantize {wl.n_ctx} K+V records, attend with {G} "
                      f"query heads; {sum(times):.1f} s timed, scaled to the full step",
            "seconds_per_step": per_step, "cpu_model": cpu_model(), "host_threads": HOST_CORES,
            "tiny_logits_s": {"all_threads": round(tiny_all, 4),
                              "one_thread": None if tiny_one is None else round(tiny_one, 4),
                              "what": "quantize 4096 fp32 keys (d=128, 3 bits) and the 64 x 4096 logits"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout "
              "(head-sharded decode, no collective) is not built here.")
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0")
        sys.exit(2)
    import torch
    import kv_cache_vector_rotation_amd as tq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    tq.lib()
    wl = synth.workload(args.workload)
    B, HQ, H, d, N = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.d, wl.n_ctx

    head, state = decode_leg(tq, torch, wl, args.steps, warmup=args.warmup, copies=args.copies)
    ms_step = state["ms_step"]
    tr = traffic_record(args.workload)
    roofline = {"bound": "hbm", "achieved": head["split_achieved_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["split_frac"], "traffic": tr["bytes_per_launch"] if tr else None,
                "kernel": "split-K pass" + (f" ({tr['kernel']})" if tr and tr.get("kernel") else ""),
                "kernel_us": head["split_kernel_us"],
                "kernel_timing": "events around replays of a graph of split-K launches, one per cache copy",
                "algorithmic_bytes": head["split_algorithmic_bytes"]}
    dims = [g for g, _ in wl.groups]
    bits = [m for _, m in wl.groups]
    result = {
        "metric": "compressed-KV decode throughput (cached tokens/s; split-K kernel vs HBM roofline)",
        "value": B * N / (ms_step / 1e3),
        "unit": "cached tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "n_q_heads": HQ, "n_kv_heads": H, "d": d,
                   "n_ctx": N, "appended_tokens": wl.n_new, "bits_per_channel": [m + 1 for m in bits],
                   "group_dims": dims, "record_bytes_per_token": head["record_bytes_per_token"],
                   "cache_copies": head["cache_copies"], "input_dtype": wl.dtype, "hip_graph": True},
        "roofline": roofline,
    }
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 device copies of {COPY_PROBE_BYTES} bytes")
        del src, dst
    if not args.no_quantize_bench:
        result["quantize"] = {"chunk": quantize_chunk_bench(tq, torch), "nn_database": quantize_nn_bench(tq, torch)}
        log(f"quantize: {result['quantize']}")
    if not (args.no_decode_legs or args.no_mixed):
        result["decode_legs"] = decode_legs(tq, torch, [w for w in DECODE_WORKLOADS if w != args.workload])
    if not args.no_bf16_baseline:
        result["bf16_baseline"] = bf16_baseline(tq, torch, wl, state["q"], ms_step)
        log(f"bf16 baseline: {result['bf16_baseline']}")
    if not args.no_chunk:
        result["chunk"] = chunk_bench(tq, torch)
        log(f"chunk: {result['chunk']}")
        result["paged"] = paged_bench(tq, torch)
        log(f"paged: {result['paged']}")
    if not args.no_variants:
        result["variants"] = variants_bench(tq, torch)
        log(f"variants: {result['variants']}")
    if not args.no_search:
        result["search"] = search_bench(tq, torch)
        log(f"search: {result['search']}")
    if args.ctx_sweep:
        result["ctx_sweep"] = ctx_sweep(tq, torch, [int(v) for v in args.ctx_sweep.split(",")])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
