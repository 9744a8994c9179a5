#!/usr/bin/env python3
"""Benchmark of the TurboQuant hot path (libtq) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

One step is one compressed-KV decode-attention call on the long-context
batched workload: batch 64 x 131072 cached tokens, 32 query / 8 KV heads,
head_dim 128, one layer, 2.5 bits per channel (keys: 32 outlier channels at
2 + 1 bits and 96 channels at 1 + 1 bits of TurboQuant_prod; values: 3 / 2
bits MSE-only; half norms per group): 84 bytes per (token, KV head), 5.64 GB
per call, resident in HBM. K calls are captured into one HIP graph and timed
with HIP events on the launch stream.

The printed JSON line also carries:
  roofline      the decode kernel's algorithmic bytes per launch / its mean
                launch time (a graph of its launches alone, found by kernel
                name), against 8 TB/s; HBM traffic from rocprofv3 counters
  cpu_baseline  the fp64 oracle on one batch element of the same workload,
                timed on this host's cores, scaled to the whole batch
  extras        the single-layer decode (batch 1, 32768 tokens; with its own
                roofline and oracle baseline), the tiny 64 x 4096 score
                matrix, prefill quantise tokens/s, vector search (batched and
                one query at a time), key/value bit allocations, the needle
                proxy, token append and paged decode, each with its oracle
                baseline where the pages' metric asks for one
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
METRIC = "compressed-KV decode attn HBM GB/s (% of peak); quantize tokens/s"
# the decode's arithmetic: query and softmax-weight digits in fp8 e4m3 times
# fp4-encoded code bit-planes on the matrix cores, fp32 accumulation
DECODE_DTYPE = "fp6e2m3 (scores) and fp8e4m3 (value sums) x fp4 mfma, fp32 accumulate"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of extras to run: single,tiny,quantize,search,bits,niah,append,step,paged")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one 256 MiB device-to-device copy (the known-size reference for the "
                        "FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/traffic_longctx_decode.json from two rocprofv3 --pmc runs of "
                        "'bench.py --no-extras --no-cpu --calibrate-copy' (FETCH_SIZE, then WRITE_SIZE) and exit")
    return p.parse_args()


class Timer:
    """HIP events on torch's current stream (the stream libtq launches on)."""

    def __init__(self):
        import torch

        self.t = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.t.cuda.synchronize()
        self.wall0 = time.perf_counter()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.t.cuda.synchronize()
        self.wall = time.perf_counter() - self.wall0
        self.ms = self.a.elapsed_time(self.b)


def dev(a, dtype=None):
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.to(dtype) if dtype is not None else t).cuda()


def blas_threads():
    """Threads numpy's BLAS runs the oracle's products on (what the oracle actually uses)."""
    try:
        from threadpoolctl import threadpool_info

        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def graph_ms(call, steps, warmup=3, warm_s=0.0):
    """Mean time per call of `steps` calls captured into one HIP graph (HIP events around one replay).

    Before capture: `warmup` calls, then more untimed calls until `warm_s`
    seconds have passed (the first few tens of long calls on a fresh GPU run
    up to 20% slower while its clocks settle).
    """
    import torch

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        call(0)
        torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                call(i)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()  # one untimed replay
    with Timer() as tm:
        graph.replay()
    res = (tm.ms / steps, side, tm.wall * 1e3 / steps)
    del graph
    return res


def _hip_runtime():
    """The HIP runtime this process already uses (the one torch loaded)."""
    import ctypes

    for line in open("/proc/self/maps"):
        if "libamdhip64.so" in line:
            return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("HIP runtime not loaded")


def kernel_only_ms(call, steps, stream, name="decode_kernel"):
    """Mean time per launch of the kernel called `name` among the launches of `call`.

    The calls are captured on `stream`; each kernel node's function handle is
    resolved to its kernel name, every node of another kernel is removed and
    the kept launches are chained one after another, so each starts when the
    previous one ends (the interval between two graph kernels is included).
    """
    import ctypes
    from ctypes import byref, c_int, c_size_t, c_uint, c_void_p

    import torch

    class KParams(ctypes.Structure):
        _fields_ = [("bx", c_uint), ("by", c_uint), ("bz", c_uint), ("extra", c_void_p), ("func", c_void_p),
                    ("gx", c_uint), ("gy", c_uint), ("gz", c_uint), ("kparams", c_void_p), ("shmem", c_uint)]

    hip = _hip_runtime()
    hip.hipKernelNameRefByPtr.restype = ctypes.c_char_p
    hip.hipKernelNameRefByPtr.argtypes = [c_void_p, c_void_p]

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: HIP error {rc}")

    s = c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    ok(hip.hipStreamBeginCapture(s, c_int(2)), "hipStreamBeginCapture")  # relaxed mode
    with torch.cuda.stream(stream):
        for i in range(steps):
            call(i)
    g = c_void_p()
    ok(hip.hipStreamEndCapture(s, byref(g)), "hipStreamEndCapture")
    try:
        nn = c_size_t(0)
        ok(hip.hipGraphGetNodes(g, None, byref(nn)), "hipGraphGetNodes")
        nodes = (c_void_p * nn.value)()
        ok(hip.hipGraphGetNodes(g, nodes, byref(nn)), "hipGraphGetNodes")
        keep, drop, names = [], [], {}
        for nd in nodes:
            t = c_int(-1)
            ok(hip.hipGraphNodeGetType(c_void_p(nd), byref(t)), "hipGraphNodeGetType")
            hit = False
            if t.value == 0:  # a kernel node: its function handle -> kernel name
                p = KParams()
                ok(hip.hipGraphKernelNodeGetParams(c_void_p(nd), byref(p)), "hipGraphKernelNodeGetParams")
                if p.func not in names:
                    nm = hip.hipKernelNameRefByPtr(c_void_p(p.func), s)
                    names[p.func] = nm.decode() if nm else ""
                hit = name in names[p.func]
            (keep if hit else drop).append(nd)
        if len(keep) != steps:
            raise RuntimeError(f"expected {steps} launches of {name}, found {len(keep)} "
                               f"(kernels: {sorted(set(names.values()))})")
        for nd in drop:
            ok(hip.hipGraphDestroyNode(c_void_p(nd)), "hipGraphDestroyNode")
        for a, b in zip(keep, keep[1:]):
            ok(hip.hipGraphAddDependencies(g, byref(c_void_p(a)), byref(c_void_p(b)), c_size_t(1)),
               "hipGraphAddDependencies")
        ex = c_void_p()
        ok(hip.hipGraphInstantiate(byref(ex), g, None, None, c_size_t(0)), "hipGraphInstantiate")
        try:
            with torch.cuda.stream(stream):
                ok(hip.hipGraphLaunch(ex, s), "hipGraphLaunch")  # one untimed replay
                with Timer() as tm:
                    ok(hip.hipGraphLaunch(ex, s), "hipGraphLaunch")
        finally:
            torch.cuda.synchronize()
            hip.hipGraphExecDestroy(ex)
    finally:
        hip.hipGraphDestroy(g)
    return tm.ms / steps


def measured_traffic(workload):
    """HBM bytes of the decode kernels from the committed counter summary of `workload`.

    profiles/traffic_<workload>.json records FETCH_SIZE and WRITE_SIZE per
    dispatch of each kernel (rocprofv3 --pmc, one counter per run), each
    scaled by what the same counter reads for a 256 MiB device copy,
    together with the SHA-256 of the kernel sources they were taken on.
    Returns None when a source has changed since (the counters no longer
    describe these kernels).
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        rec = json.load(open(path))
        for rel, digest in rec["source_sha256"].items():
            if hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest() != digest:
                return None
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    per = [v for k, v in rec.get("per_kernel", {}).items() if k.startswith("decode_kernel")]
    if len(per) != 1:
        return None
    return {"call": rec.get("bytes_per_call"), "decode_kernel": per[0]["fetch_bytes"] + per[0]["write_bytes"]}


TRAFFIC_SOURCES = ["decode_tq_quantize_amd/csrc/decode_mfma.hip", "decode_tq_quantize_amd/csrc/internal.h"]


def traffic_summary(fetch_dir, write_dir):
    """HBM bytes per dispatch of the long-context decode kernels from two
    rocprofv3 counter runs (csv output), written to
    profiles/traffic_longctx_decode.json.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the
    same counter reads for the 256 MiB device copy --calibrate-copy runs
    first (the first copy dispatch of the run: later copies, of other sizes,
    are the inputs' set-up). The median over a kernel's dispatches is kept
    (the one quality call that also writes the score matrix is an outlier).
    """
    import collections
    import csv
    import glob
    import hashlib
    import re
    import statistics

    def load(folder, counter):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    per[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        # the calibration copy: the run's first copy dispatch
        copies = [(d, v) for k, dv in per.items() if "copy" in k.lower() for d, v in dv.items()]
        return {k: list(v.values()) for k, v in per.items()}, min(copies)[1]

    (F, fcopy), (W, wcopy) = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_kib = (256 << 20) / 1024
    ff, wf = copy_kib / fcopy, copy_kib / wcopy

    def short(k):
        for s in ("qfused_kernel", "qtransform_kernel", "combine_kernel"):
            if s in k:
                return s
        return "decode_kernel" if "decode_kernel<" in k else None

    per = {}
    for k in F:
        s = short(k)
        if s is None or k not in W:
            continue
        fk, wk = statistics.median(F[k]), statistics.median(W[k])
        m = re.search(r"\w+_kernel(<[^>]*>)?", k)
        per[s] = {"kernel": m.group(0) if m else k, "fetch_kib": round(fk, 2),
                  "write_kib": round(wk, 2), "fetch_bytes": int(round(fk * 1024 * ff)),
                  "write_bytes": int(round(wk * 1024 * wf)), "dispatches": len(F[k])}
    n = LC["B"] * LC["Hkv"] * LC["T"]
    kv_bytes = n * LC_BYTES_PER_TOKEN_HEAD
    rec = {"what": "HBM bytes per dispatch of the long-context decode call (batch 64 x 131072 tokens, 32 q / 8 KV "
                   "heads, head_dim 128, 2.5 bits per channel): rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by "
                   "its reading for a 256 MiB device copy; median over dispatches",
           "commands": ["rocprofv3 --output-format csv --pmc FETCH_SIZE -d <fetch_dir> -o fetch -- python3 bench.py "
                        "--no-extras --no-cpu --steps 6 --warmup 1 --calibrate-copy",
                        "rocprofv3 --output-format csv --pmc WRITE_SIZE -d <write_dir> -o write -- python3 bench.py "
                        "--no-extras --no-cpu --steps 6 --warmup 1 --calibrate-copy",
                        "python3 bench.py --traffic-summary <fetch_dir> <write_dir>"],
           "calibration": {"copy_bytes": 256 << 20, "fetch_size_kib": round(fcopy, 4), "write_size_kib": round(wcopy, 4),
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "per_kernel": per,
           "bytes_per_call": sum(v["fetch_bytes"] + v["write_bytes"] for v in per.values()),
           "algorithmic_bytes_decode_kernel": kv_bytes,
           "algorithmic_bytes_per_call": kv_bytes + LC["B"] * LC["Hq"] * LC["d"] * (2 + 4),
           "source_sha256": {rel: hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()
                             for rel in TRAFFIC_SOURCES}}
    if "decode_kernel" in per:
        dk = per["decode_kernel"]
        rec["decode_kernel_traffic_over_algorithmic"] = round((dk["fetch_bytes"] + dk["write_bytes"]) / kv_bytes, 4)
    out = os.path.join(ROOT, "profiles", "traffic_longctx_decode.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def roofline_block(kernel_bytes, kernel_ms, call_bytes, call_ms, traffic, kernel_desc):
    ach = kernel_bytes / (kernel_ms * 1e-3) / 1e9
    call = call_bytes / (call_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic["decode_kernel"] if traffic else None,
            "kernel": kernel_desc, "bytes_per_launch": kernel_bytes, "us_per_launch": round(kernel_ms * 1e3, 3),
            "whole_call": {"kernels": "everything one tq_decode_attn call launches",
                           "achieved": round(call, 2), "frac": round(call / HBM_PEAK_GBS, 4),
                           "bytes_per_call": call_bytes, "us_per_call": round(call_ms * 1e3, 3),
                           "traffic": traffic["call"] if traffic else None}}


# --------------------------------------------------------------------------
# the headline: long-context batched decode
# --------------------------------------------------------------------------

LC = dict(B=64, Hq=32, Hkv=8, T=131072, d=128)
LC_GROUPS_K = [(0, 32, 2, True), (32, 96, 1, True)]     # (first channel, channels, MSE bits, QJL sign)
LC_GROUPS_V = [(0, 32, 3, False), (32, 96, 2, False)]
LC_BYTES_PER_TOKEN_HEAD = 84


def _lc_matrices(gi, gd, prod, stream):
    import synth

    seed = 40 + gi + 10 * stream
    R = synth.haar_orthogonal(gd, seed)
    S = synth.gaussian_matrix(gd, gd, seed) if prod else None
    return R, S


def longctx_decode(args):
    """Batch 64 x 131072 tokens; returns timings plus what the CPU baseline needs."""
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    from synth import device as sdev

    B, Hq, Hkv, T, d = LC["B"], LC["Hq"], LC["Hkv"], LC["T"], LC["d"]
    n = B * Hkv * T
    keep, descs, host = [], {}, {}
    cache_q = []  # the cache's quantisation, one call per channel group (timed once each)
    for name, groups, layout, stream in (("k", LC_GROUPS_K, tq.TQ_LAYOUT_KEYS, 11),
                                         ("v", LC_GROUPS_V, tq.TQ_LAYOUT_VALUES, 12)):
        log(f"longctx: generating {name} ({n * d * 2 / 1e9:.1f} GB bf16), outlier channels first")
        X = sdev.kv_with_outliers(B, Hkv, T, d, 0, 1.0, seed=4, stream=stream)
        X[..., :32] *= 10  # the 32 outlier channels, already permuted to the front
        X = X.view(n, d)
        host[name] = X[:Hkv * T].float().cpu().numpy()  # batch element 0 (rows (0, g, t))
        gl = []
        for gi, (ch, gd, bits, prod) in enumerate(groups):
            R, S = _lc_matrices(gi, gd, prod, stream)
            R_t, S_t = dev(R), (dev(S) if prod else None)
            var = tq.TQ_PROD if prod else tq.TQ_MSE
            q = tq.tq_quantizer_init(gd, bits, var, R_t, S_t)
            if prod:
                SR_t = torch.empty(tq.tq_fold_bytes(gd) // 4, dtype=torch.float32, device="cuda")
                tq.tq_quantizer_fold(q, SR_t)
                keep.append(SR_t)
            pk = torch.empty(tq.tq_packed_bytes(gd, bits, var, layout, n) // 4, dtype=torch.int32, device="cuda")
            nr = torch.empty(n, dtype=torch.int16, device="cuda")
            rr = torch.empty(n, dtype=torch.int16, device="cuda") if prod else None
            with Timer() as tm:
                tq.tq_quantize_kv(q, layout, tq.TQ_BF16, X[:, ch:], n, d, pk, nr, rr)
            # HBM bytes: the group's bf16 channels read, its bit planes and fp16 norms written
            qbytes = n * gd * 2 + pk.numel() * 4 + n * 2 * (2 if prod else 1)
            cache_q.append({"group": f"{'K' if name == 'k' else 'V'} channels {ch}..{ch + gd - 1}, {bits}"
                                     f"{'+1' if prod else ''} bits", "vectors": n, "ms": round(tm.ms, 3),
                            "vectors_per_s": round(n / (tm.ms * 1e-3), 1),
                            "hbm_gbs": round(qbytes / (tm.ms * 1e-3) / 1e9, 1),
                            "hbm_roofline_frac": round(qbytes / (tm.ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            keep += [R_t, S_t, pk, nr, rr]
            gl.append(tq.make_group(q, ch, pk, nr, rr, T))
        torch.cuda.synchronize()
        del X
        torch.cuda.empty_cache()
        descs[name] = tq.make_desc(gl)
    q_t = torch.randn((B, Hq, d), generator=sdev.generator(4, 13), device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    wsb = tq.tq_decode_workspace_bytes(descs["k"], descs["v"], B, Hq, Hkv, T)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)

    def call(i):
        tq.tq_decode_attn(descs["k"], descs["v"], q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, scale, out, None, ws, wsb)

    log(f"longctx: {args.steps} calls in one graph")
    ms, side, wall_ms = graph_ms(call, args.steps, args.warmup, warm_s=0.5)
    dk_ms = kernel_only_ms(call, args.steps, side)
    kv_bytes = n * LC_BYTES_PER_TOKEN_HEAD
    call_bytes = kv_bytes + B * Hq * d * (2 + 4)
    log(f"longctx: {ms:.4f} ms/call ({call_bytes / ms / 1e6:.1f} GB/s); decode kernel {dk_ms:.4f} ms "
        f"({kv_bytes / dk_ms / 1e6:.1f} GB/s)")
    # quality (not parity): query heads 0..3 (KV head 0, batch 0) against exact
    # fp64 attention on the bf16 K and V; one more (untimed) call returns the
    # raw score estimates
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    tq.tq_decode_attn(descs["k"], descs["v"], q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, scale, out, scores, ws, wsb)
    torch.cuda.synchronize()
    G = Hq // Hkv
    qs = q_t[0, :G].float().cpu().double().numpy()
    o_gpu = out[0, :G].cpu().double().numpy()
    s_gpu = scores[0, :G].cpu().double().numpy().T  # [T, G]
    del scores
    kb, vb = host["k"][:T].astype(np.float64), host["v"][:T].astype(np.float64)
    s_ex = kb @ qs.T
    lg = s_ex * scale
    pw = np.exp(lg - lg.max(axis=0))
    o_ex = (pw.T @ vb) / pw.sum(axis=0)[:, None]
    rel = np.linalg.norm(o_gpu - o_ex, axis=1) / np.linalg.norm(o_ex, axis=1)
    s_rel = np.linalg.norm(s_gpu - s_ex, axis=0) / np.linalg.norm(s_ex, axis=0)
    s_cos = (s_gpu * s_ex).sum(axis=0) / (np.linalg.norm(s_gpu, axis=0) * np.linalg.norm(s_ex, axis=0))
    bf16_bytes = n * d * 2 * 2
    res = {"per_call_ms": ms, "wall_ms": wall_ms, "call_bytes": call_bytes, "dk_ms": dk_ms, "kv_bytes": kv_bytes,
           "extras": {"cache_quantize": cache_q,
                      "bf16_attention_roofline_ms": round(bf16_bytes / HBM_PEAK_GBS / 1e6, 4),
                      "speedup_vs_bf16_roofline": round(bf16_bytes / HBM_PEAK_GBS / 1e6 / ms, 3),
                      "quality_vs_exact_bf16_attention": {
                          "sample": "batch 0, query heads 0-3 (KV head 0), 131072 tokens",
                          "score_rel_error": round(float(s_rel.mean()), 4),
                          "score_cosine": round(float(s_cos.mean()), 4),
                          "output_rel_error": round(float(rel.mean()), 4)}},
           "oracle": (host, q_t[:1].float().cpu().numpy())}
    del keep, descs, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline_longctx(oracle_inputs, call_bytes):
    """The oracle's decode of batch element 0 (8 KV heads, 32 query heads, 131072 tokens), x 64."""
    import numpy as np

    from oracle import tq as otq

    host, qry = oracle_inputs
    Hkv, T, d = LC["Hkv"], LC["T"], LC["d"]
    log("cpu baseline (long-context): oracle quantisation of batch element 0 (untimed)")
    groups = {}
    for name, specs, stream in (("k", LC_GROUPS_K, 11), ("v", LC_GROUPS_V, 12)):
        X = host[name].astype(np.float64).reshape(1, Hkv, T, d)
        gl = []
        for gi, (ch, gd, bits, prod) in enumerate(specs):
            R, S = _lc_matrices(gi, gd, prod, stream)
            oq = otq.make_quantizer(gd, bits, prod, R, S)
            gl.append(otq.Group(ch, oq, otq.quantize(X[..., ch:ch + gd], oq)))
        groups[name] = gl
    threads = blas_threads()
    log(f"cpu baseline (long-context): oracle decode on {threads} threads")
    t0 = time.perf_counter()
    otq.decode_attention(qry.astype(np.float64), groups["k"], groups["v"], Hkv)
    dt = time.perf_counter() - t0
    per_call = dt * LC["B"]
    return {"value": round(call_bytes / per_call / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"batch element 0 of 64 (8 KV heads, 32 query heads, 131072 tokens, both channel groups), "
                      f"{dt:.2f} s, scaled x64 to the whole call; codes from the oracle's own quantiser (untimed)"}


# --------------------------------------------------------------------------
# extras
# --------------------------------------------------------------------------

def single_layer_decode(steps=200, copies=24, cpu=True):
    """Batch 1, 32 q / 8 KV heads, d = 128, 32768 tokens; K 3+1-bit prod, V 3-bit MSE."""
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth

    B, Hq, Hkv, T, d = 1, 32, 8, 32768, 128
    n = B * Hkv * T
    log("single-layer decode: generating inputs")
    K = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, 2, synth.STREAM_DATA, synth.STREAM_OUTLIER)
    V = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, 2, synth.STREAM_NORM, synth.STREAM_R_V)
    qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.rng(2, synth.STREAM_QUERY).standard_normal(
        (B, Hq, d)).astype(np.float32)))
    Rk, Sk = synth.haar_orthogonal(d, 2), synth.gaussian_matrix(d, d, 2)
    Rv = synth.haar_orthogonal(d, 2, synth.STREAM_R_V)
    Rk_t, Sk_t, Rv_t = dev(Rk), dev(Sk), dev(Rv)
    qk = tq.tq_quantizer_init(d, 3, tq.TQ_PROD, Rk_t, Sk_t)
    SRk = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
    tq.tq_quantizer_fold(qk, SRk)  # S R once per quantiser (setup, untimed)
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
    kp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, n) // 4, dtype=torch.int32, device="cuda")
    vp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n) // 4, dtype=torch.int32, device="cuda")
    kn, kr, vn = (torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(3))
    tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, dev(K.reshape(n, d), torch.bfloat16), n, d, kp, kn, kr)
    tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, dev(V.reshape(n, d), torch.bfloat16), n, d, vp, vn)
    # copies of the 31 MB cache rotated inside the graph, so that no call
    # finds its cache in the 256 MB last-level cache
    cps = []
    for _ in range(copies):
        bufs = [x.clone() for x in (kp, kn, kr, vp, vn)]
        kd = tq.make_desc([tq.make_group(qk, 0, bufs[0], bufs[1], bufs[2], T)])
        vd = tq.make_desc([tq.make_group(qv, 0, bufs[3], bufs[4], None, T)])
        cps.append((bufs, kd, vd))
    q_t = dev(qry, torch.bfloat16)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    wsb = tq.tq_decode_workspace_bytes(cps[0][1], cps[0][2], B, Hq, Hkv, T)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)

    def call(i):
        _, kd, vd = cps[i % len(cps)]
        tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, scale, out, None, ws, wsb)

    ms, side, _ = graph_ms(call, steps)
    dk_ms = kernel_only_ms(call, steps, side)
    kv_bytes = n * 118
    call_bytes = kv_bytes + B * Hq * d * (2 + 4)
    res = {"workload": "single-layer decode, Llama-3.1-8B shape: batch 1, 32 q / 8 KV heads, d=128, 32768 tokens; "
                       f"K 3+1-bit prod, V 3-bit MSE; 118 B per token-head; {copies} cache copies rotated",
           "us_per_call": round(ms * 1e3, 3), "gbs": round(call_bytes / ms / 1e6, 1),
           "roofline": roofline_block(kv_bytes, dk_ms, call_bytes, ms, measured_traffic("single_layer_decode"),
                                      "decode_kernel")}
    log(f"single-layer decode: {res}")
    if cpu:
        from oracle import tq as otq

        oqk = otq.make_quantizer(d, 3, True, Rk, Sk)
        oqv = otq.make_quantizer(d, 3, False, Rv)
        ck, cv = otq.quantize(K, oqk), otq.quantize(V, oqv)
        threads = blas_threads()
        t0 = time.perf_counter()
        reps = 0
        while True:
            otq.decode_attention(qry.astype(np.float64), [otq.Group(0, oqk, ck)], [otq.Group(0, oqv, cv)], Hkv)
            reps += 1
            if time.perf_counter() - t0 > 8.0 and reps >= 2:
                break
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(call_bytes / dt / 1e9, 5), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "sample": f"the full call, {reps} repetition(s), {dt:.2f} s each; "
                                                           "codes from the oracle's own quantiser (untimed)"}
    res["oracle_inputs"] = (K, V, qry, Rk, Sk, Rv)
    del cps, ws
    torch.cuda.empty_cache()
    return res


def tiny_score_matrix(steps=200, cpu=True):
    """4096 unit keys, d = 128, 64 queries; PROD b = 2, 3, 4; the 64 x 4096 score matrix."""
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth

    d, N, Q = 128, 4096, 64
    keys = synth.unit_gaussian(N, d, 0)
    qry = synth.unit_gaussian(Q, d, 0, synth.STREAM_QUERY)
    Vx = synth.unit_gaussian(N, d, 0, synth.STREAM_NORM)
    R, S = synth.haar_orthogonal(d, 0), synth.gaussian_matrix(d, d, 0)
    Rv = synth.haar_orthogonal(d, 0, synth.STREAM_R_V)
    R_t, S_t, Rv_t = dev(R), dev(S), dev(Rv)
    rows = []
    for b in (2, 3, 4):
        qk = tq.tq_quantizer_init(d, b - 1, tq.TQ_PROD, R_t, S_t)
        SR = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
        tq.tq_quantizer_fold(qk, SR)
        qv = tq.tq_quantizer_init(d, 2, tq.TQ_MSE, Rv_t)
        kp = torch.empty(tq.tq_packed_bytes(d, b - 1, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, N) // 4, dtype=torch.int32,
                         device="cuda")
        vp = torch.empty(tq.tq_packed_bytes(d, 2, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, N) // 4, dtype=torch.int32,
                         device="cuda")
        kn, kr, vn = (torch.empty(N, dtype=torch.int16, device="cuda") for _ in range(3))
        tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_F32, dev(keys), N, d, kp, kn, kr)
        tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_F32, dev(Vx), N, d, vp, vn)
        kd = tq.make_desc([tq.make_group(qk, 0, kp, kn, kr, N)])
        vd = tq.make_desc([tq.make_group(qv, 0, vp, vn, None, N)])
        q_t = dev(qry.reshape(1, Q, d))
        out = torch.empty((1, Q, d), dtype=torch.float32, device="cuda")
        sc = torch.empty((1, Q, N), dtype=torch.float32, device="cuda")
        wsb = tq.tq_decode_workspace_bytes(kd, vd, 1, Q, 1, N)
        ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")

        def call(i):
            tq.tq_decode_attn(kd, vd, q_t, tq.TQ_F32, 1, Q, 1, N, None, 1 / math.sqrt(d), out, sc, ws, wsb)

        ms, _, _ = graph_ms(call, steps)
        row = {"bits": b, "us_per_call": round(ms * 1e3, 3), "scores_per_s": round(Q * N / ms * 1e3, 1)}
        if cpu:
            from threadpoolctl import threadpool_limits

            from oracle import tq as otq

            oq = otq.make_quantizer(d, b - 1, True, R, S)
            codes = otq.quantize(keys.astype(np.float64), oq)
            for label, lim in (("oracle_1_core", 1), ("oracle_all_cores", None)):
                with threadpool_limits(limits=lim):
                    threads = blas_threads()
                    t0 = time.perf_counter()
                    reps = 0
                    while time.perf_counter() - t0 < 1.0 or reps < 3:
                        otq.estimate_ip(qry.astype(np.float64), codes, oq)
                        reps += 1
                    dt = (time.perf_counter() - t0) / reps
                row[label] = {"seconds": round(dt, 5), "scores_per_s": round(Q * N / dt, 1), "cores": threads}
        rows.append(row)
        log(f"tiny score matrix: {row}")
    return {"workload": "4096 keys d=128 and 64 queries, N(0,I) unit-normalised, TurboQuant_prod b=2,3,4; the 64 x "
                        "4096 score matrix through tq_decode_attn's score output (Hkv=1, Hq=64); launch-bound, "
                        "parity only (no roofline)", "rows": rows}


def quantize_prefill(steps=2, cpu=True):
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    L, S, Tq, H, d = 32, 16, 8192, 8, 128
    n = S * Tq * H
    log("quantize: generating 17.2 GB of bf16 K/V on the device")
    X = torch.empty((L, 2, n, d), dtype=torch.bfloat16, device="cuda")
    for l in range(L):
        for t in range(2):
            sdev.lognormal_norm_vectors(n, d, seed=1000 + 2 * l + t, out=X[l, t])
    Rk, Sk = synth.haar_orthogonal(d, 3), synth.gaussian_matrix(d, d, 3)
    Rv = synth.haar_orthogonal(d, 3, synth.STREAM_R_V)
    Rk_t, Sk_t, Rv_t = dev(Rk), dev(Sk), dev(Rv)
    qk = tq.tq_quantizer_init(d, 2, tq.TQ_PROD, Rk_t, Sk_t)
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
    kb = tq.tq_packed_bytes(d, 2, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, n)
    vb = tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n)
    kp = torch.empty((L, kb // 4), dtype=torch.int32, device="cuda")
    vp = torch.empty((L, vb // 4), dtype=torch.int32, device="cuda")
    kn = torch.empty((L, n), dtype=torch.int16, device="cuda")
    kr = torch.empty((L, n), dtype=torch.int16, device="cuda")
    vn = torch.empty((L, n), dtype=torch.int16, device="cuda")

    def step():
        for l in range(L):
            tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, X[l, 0], n, d, kp[l], kn[l], kr[l])
            tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, X[l, 1], n, d, vp[l], vn[l])

    step()
    with Timer() as tm:
        for _ in range(steps):
            step()
    sec = tm.ms * 1e-3 / steps
    tokens = S * Tq
    flops = tokens * L * H * (2 * 2 * d * d + 2 * d * d)
    bytes_ = tokens * L * H * (2 * d * 2 + (3 * 16 + 4) + (3 * 16 + 2))
    res = {"tokens_per_s": round(tokens / sec, 1), "ms_per_step": round(sec * 1e3, 3),
           "workload": "16 seq x 8192 tok x 32 layers x 8 KV heads, d=128, bf16; K 3-bit prod, V 3-bit MSE",
           "achieved_tflops": round(flops / sec / 1e12, 2), "hbm_gbs": round(bytes_ / sec / 1e9, 1),
           # the products run on the bf16 matrix cores (operands split into
           # bf16 high and low parts), so their peak is the bf16 one
           "flops_roofline_frac_bf16_mfma": round(flops / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
           "hbm_roofline_frac": round(bytes_ / sec / 1e9 / HBM_PEAK_GBS, 4)}
    if cpu:
        from oracle import tq as otq

        # one (layer, KV head) slice: the 131072 vectors of layer 0's first KV
        # head per tensor (vector (s, t, h) is row (s * 8192 + t) * 8 + h)
        xs = [X[0, t].view(S * Tq, H, d)[:, 0].float().cpu().numpy().astype(np.float64) for t in (0, 1)]
        oqk = otq.make_quantizer(d, 2, True, Rk, Sk)
        oqv = otq.make_quantizer(d, 3, False, Rv)
        threads = blas_threads()
        t0 = time.perf_counter()
        ck = otq.quantize(xs[0], oqk)
        otq.pack(ck.idx, ck.z, 2, "keys")
        cv = otq.quantize(xs[1], oqv)
        otq.pack(cv.idx, None, 3, "values")
        dt = time.perf_counter() - t0
        del ck, cv
        res["cpu_baseline"] = {"value": round(tokens / (dt * L * H), 2), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"1 layer x 1 KV head (131072 key and 131072 value vectors), {dt:.2f} s, "
                                         f"scaled x256 to 32 layers x 8 KV heads"}
    del X
    torch.cuda.empty_cache()
    return res


def vector_search(steps=2, stream_steps=50, cpu=True):
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    N, d, Q, k = 1 << 20, 1536, 1024, 10
    log("search: generating the 1M x 1536 database")
    db, means = sdev.gaussian_mixture(N, d, 256, seed=5, stream=0)
    qs, _ = sdev.gaussian_mixture(Q, d, 256, seed=5, stream=1, means=means)
    R, S = synth.haar_orthogonal(d, 5), synth.gaussian_matrix(d, d, 5)
    R_t, S_t = dev(R), dev(S)
    q = tq.tq_quantizer_init(d, 3, tq.TQ_PROD, R_t, S_t)
    pk = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, N) // 4, dtype=torch.int32, device="cuda")
    nr = torch.empty(N, dtype=torch.int16, device="cuda")
    rr = torch.empty(N, dtype=torch.int16, device="cuda")
    tq.tq_quantize_kv(q, tq.TQ_LAYOUT_KEYS, tq.TQ_F32, db, N, d, pk, nr, rr)
    with Timer() as tq_build:
        tq.tq_quantize_kv(q, tq.TQ_LAYOUT_KEYS, tq.TQ_F32, db, N, d, pk, nr, rr)
    g = tq.make_group(q, 0, pk, nr, rr, 0)
    wsb = tq.tq_search_workspace_bytes(g, N, Q, k)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    oi = torch.empty((Q, k), dtype=torch.int64, device="cuda")
    osc = torch.empty((Q, k), dtype=torch.float32, device="cuda")
    tq.tq_search_topk(g, N, qs, Q, k, oi, osc, ws, wsb)
    with Timer() as tm:
        for _ in range(steps):
            tq.tq_search_topk(g, N, qs, Q, k, oi, osc, ws, wsb)
    sec = tm.ms * 1e-3 / steps
    # one query at a time (streaming): the whole database is read per query
    wsb1 = tq.tq_search_workspace_bytes(g, N, 1, k)
    ws1 = torch.empty(wsb1 // 4 + 4, dtype=torch.float32, device="cuda")
    oi1 = torch.empty((1, k), dtype=torch.int64, device="cuda")
    os1 = torch.empty((1, k), dtype=torch.float32, device="cuda")

    def one(i):
        tq.tq_search_topk(g, N, qs[i % Q:i % Q + 1], 1, k, oi1, os1, ws1, wsb1)

    ms1, _, _ = graph_ms(one, stream_steps)
    db_bytes = N * (4 * d // 8 + 4)
    # recall@10 against exact fp64 inner products on a 64-query sample
    sample = 64
    exact = (qs[:sample].double() @ db.double().T)
    top = torch.topk(exact, k, dim=1).indices.cpu().numpy()
    got = oi[:sample].cpu().numpy()
    rec = float(np.mean([len(set(got[i].tolist()) & set(top[i].tolist())) / k for i in range(sample)]))
    del exact
    # estimator work: both sums, 2 d multiply-adds per (query, vector)
    flops = 2.0 * Q * N * 2 * d
    # what the bf16 matrix cores execute: per coordinate 4 Walsh terms x 2
    # operand halves + 3 QJL products = 11 multiply-adds per (query, vector)
    mfma_flops = 2.0 * 11 * Q * N * d
    res = {"qps": round(Q / sec, 1), "ms_per_batch": round(sec * 1e3, 3), "recall_at_10": round(rec, 4),
           "estimator_tflops": round(flops / sec / 1e12, 2),
           "mfma_bf16_tflops_executed": round(mfma_flops / sec / 1e12, 2),
           "mfma_bf16_roofline_frac": round(mfma_flops / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
           "streaming": {"qps": round(1e3 / ms1, 1), "us_per_query": round(ms1 * 1e3, 2),
                         "db_bytes_per_query": db_bytes,
                         "hbm_gbs": round(db_bytes / ms1 / 1e6, 1),
                         "hbm_roofline_frac": round(db_bytes / ms1 / 1e6 / HBM_PEAK_GBS, 4),
                         "how": f"{stream_steps} single-query calls in one graph"},
           "db_quantize_ms": round(tq_build.ms, 3),
           "workload": "1M x 1536 fp32 256-component Gaussian mixture, unit-normalised; 1024 queries; "
                       "4-bit prod (3+1) codes; top-10"}
    log(f"search: {res}")
    if cpu:
        from oracle import tq as otq

        # the oracle searches the GPU's own codes (unpacked on the host, untimed)
        words = pk.cpu().numpy().view(np.uint32)
        idx, z = otq.unpack(words, N, d, 3, True, "keys")
        codes = otq.Codes(idx, z, None, None, nr.cpu().numpy().view(np.float16), rr.cpu().numpy().view(np.float16),
                          None, None)
        del words
        oq = otq.make_quantizer(d, 3, True, R, S)
        yq = qs[:64].cpu().numpy().astype(np.float64)
        threads = blas_threads()
        t0 = time.perf_counter()
        otq.search_topk(yq, codes, oq, k)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(Q / (dt * 16), 3), "unit": "QPS", "cores": threads, "kind": "oracle",
                               "sample": f"64 of the 1024 queries against the whole database, {dt:.2f} s, "
                                         f"scaled x16; the GPU's codes unpacked on the host (untimed)"}
        del idx, z, codes
    del db, pk, ws
    torch.cuda.empty_cache()
    return res


# key / value bit allocations at the single-layer shape: (name, key MSE bits,
# key has the QJL sketch, value bits)
ALLOCATIONS = [
    ("keys 3+1 prod, values 3 (headline)", 3, True, 3),
    ("keys 4 MSE-only, values 3", 4, False, 3),
    ("keys 3 MSE-only, values 3", 3, False, 3),
    ("keys 3+1 prod, values 2", 3, True, 2),
    ("keys 2+1 prod, values 2", 2, True, 2),
]


def bit_allocations(inputs, steps=100, copies=12):
    """Decode rate and attention quality of several key/value bit allocations.

    Same single-layer shape and inputs as the headline (batch 1, 32 q / 8 KV
    heads, head_dim 128, 32768 tokens, bf16 K and V with outlier channels).
    Each allocation quantises K and V with libtq (untimed), rotates `copies`
    copies of its cache inside one captured graph, and reports per-call and
    decode-kernel rates against its own algorithmic bytes; quality compares
    KV head 0's four query heads with exact fp64 attention on the bf16 K and V.
    """
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth

    K, V, qry, Rk, Sk, Rv = inputs
    B, Hq, Hkv, T, d = 1, 32, 8, 32768, 128
    n = B * Hkv * T
    Kt = dev(K.reshape(n, d), torch.bfloat16)
    Vt = dev(V.reshape(n, d), torch.bfloat16)
    Kb = Kt[:T].double().cpu().numpy()  # (b 0, KV head 0) rows of the bf16 inputs
    Vb = Vt[:T].double().cpu().numpy()
    q_t = dev(qry, torch.bfloat16)
    G = Hq // Hkv
    qs = q_t[0, :G].double().cpu().numpy()
    s_ex = Kb @ qs.T  # [T, G]
    lg = s_ex / math.sqrt(d)
    pw = np.exp(lg - lg.max(axis=0))
    o_ex = (pw.T @ Vb) / pw.sum(axis=0)[:, None]
    Rk_t, Sk_t, Rv_t = dev(Rk), dev(Sk), dev(Rv)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    res = []
    for name, kb, kprod, vb in ALLOCATIONS:
        kvar = tq.TQ_PROD if kprod else tq.TQ_MSE
        qk = tq.tq_quantizer_init(d, kb, kvar, Rk_t, Sk_t if kprod else None)
        SRk = None
        if kprod:
            SRk = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
            tq.tq_quantizer_fold(qk, SRk)
        qv = tq.tq_quantizer_init(d, vb, tq.TQ_MSE, Rv_t)
        kp = torch.empty(tq.tq_packed_bytes(d, kb, kvar, tq.TQ_LAYOUT_KEYS, n) // 4, dtype=torch.int32, device="cuda")
        vp = torch.empty(tq.tq_packed_bytes(d, vb, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n) // 4, dtype=torch.int32,
                         device="cuda")
        kn, vn = (torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(2))
        kr = torch.empty(n, dtype=torch.int16, device="cuda") if kprod else None
        tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, Kt, n, d, kp, kn, kr)
        tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, Vt, n, d, vp, vn)
        cps = []
        for c in range(copies):
            bufs = [x.clone() if x is not None else None for x in (kp, kn, kr, vp, vn)]
            kd = tq.make_desc([tq.make_group(qk, 0, bufs[0], bufs[1], bufs[2], T)])
            vd = tq.make_desc([tq.make_group(qv, 0, bufs[3], bufs[4], None, T)])
            cps.append((bufs, kd, vd))
        wsb = tq.tq_decode_workspace_bytes(cps[0][1], cps[0][2], B, Hq, Hkv, T)
        ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")

        def call(i):
            _, kd, vd = cps[i % len(cps)]
            tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, scale, out, None, ws, wsb)

        ms, side, _ = graph_ms(call, steps)
        dk_ms = kernel_only_ms(call, steps, side)
        kv_bytes = n * ((kb + kprod) * (d // 8) + 2 + 2 * kprod + vb * (d // 8) + 2)
        call_bytes = kv_bytes + B * Hq * d * (2 + 4)
        scores = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
        _, kd, vd = cps[0]
        tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, scale, out, scores, ws, wsb)
        torch.cuda.synchronize()
        s_gpu = scores[0, :G].double().cpu().numpy().T
        o_gpu = out[0, :G].double().cpu().numpy()
        s_rel = np.linalg.norm(s_gpu - s_ex, axis=0) / np.linalg.norm(s_ex, axis=0)
        o_rel = np.linalg.norm(o_gpu - o_ex, axis=1) / np.linalg.norm(o_ex, axis=1)
        top1 = float(np.mean(np.argmax(s_gpu, axis=0) == np.argmax(s_ex, axis=0)))
        res.append({"allocation": name, "bytes_per_token_head": kv_bytes // n,
                    "bits_per_channel": round(8 * (kv_bytes // n) / (2 * d), 3),
                    "us_per_call": round(ms * 1e3, 3), "call_gbs": round(call_bytes / ms / 1e6, 1),
                    "decode_kernel_us": round(dk_ms * 1e3, 3), "decode_kernel_gbs": round(kv_bytes / dk_ms / 1e6, 1),
                    "decode_kernel_hbm_frac": round(kv_bytes / dk_ms / 1e6 / HBM_PEAK_GBS, 4),
                    "score_rel_error": round(float(s_rel.mean()), 4),
                    "output_rel_error": round(float(o_rel.mean()), 4),
                    "top1_token_agreement": top1})
        log(f"bit allocation {res[-1]}")
        del cps, ws, scores, kp, vp, kn, vn, kr, SRk
        torch.cuda.empty_cache()
    # the section 4.5 rule applied to these inputs' median key and value norms
    kn_med = float(np.median(np.linalg.norm(Kb, axis=1)))
    vn_med = float(np.median(np.linalg.norm(Vb, axis=1)))
    cls, kbits, vbits = tq.tq_kv_bit_allocation(kn_med, vn_med)
    policy = {"median_key_norm": round(kn_med, 3), "median_value_norm": round(vn_med, 3),
              "ratio": round(kn_med / vn_med, 3), "class": ["uniform", "asymmetric", "mixed"][cls],
              "key_bits": kbits, "value_bits": vbits}
    return {"workload": "single-layer decode shape (batch 1, 32 q / 8 KV heads, d=128, 32768 tokens), same bf16 "
                        "inputs as the headline; quality on KV head 0's 4 query heads against exact fp64 attention",
            "norm_ratio_policy": policy, "allocations": res}


def append_step(steps=200):
    """Latency of appending one decoded token per (sequence, KV head) to the cache.

    Batch 64 x 8 KV heads, d = 128 (the long-context decode's sequences, one
    new token each): K as 3+1-bit prod and V as 3-bit MSE, each one
    tq_append_kv call writing 512 rows of a 4096-token-per-head cache; the
    two calls of a step are captured into one graph with the step's rows
    advancing by one token per step.
    """
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    B, Hkv, d, T = 64, 8, 128, 4096
    Rk_t, Sk_t = dev(synth.haar_orthogonal(d, 5)), dev(synth.gaussian_matrix(d, d, 5))
    Rv_t = dev(synth.haar_orthogonal(d, 5, synth.STREAM_R_V))
    qk = tq.tq_quantizer_init(d, 3, tq.TQ_PROD, Rk_t, Sk_t)
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
    C = B * Hkv * T
    kp = torch.zeros(tq.tq_packed_bytes(d, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, C) // 4, dtype=torch.int32, device="cuda")
    vp = torch.zeros(tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, C) // 4, dtype=torch.int32,
                     device="cuda")
    kn, kr, vn = (torch.zeros(C, dtype=torch.int16, device="cuda") for _ in range(3))
    xk = sdev.kv_with_outliers(1, Hkv, B, d, 4, 10.0, seed=5, stream=31).view(B * Hkv, d)
    xv = sdev.kv_with_outliers(1, Hkv, B, d, 4, 10.0, seed=5, stream=32).view(B * Hkv, d)
    base = torch.arange(B * Hkv, device="cuda", dtype=torch.int64) * T
    rows = [base + (1000 + i) for i in range(steps)]  # token 1000 + i of every (sequence, head)
    n = B * Hkv

    def call(i):
        r = rows[i % len(rows)]
        tq.tq_append_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, xk, n, d, r, C, kp, kn, kr)
        tq.tq_append_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, xv, n, d, r, C, vp, vn)

    ms, _, _ = graph_ms(call, steps)

    def call_pair(i):
        r = rows[i % len(rows)]
        tq.tq_append_kv_pair(qk, qv, tq.TQ_BF16, xk, xv, n, d, d, r, C, kp, kn, kr, vp, vn)

    ms_pair, _, _ = graph_ms(call_pair, steps)
    return {"us_per_step": round(ms_pair * 1e3, 3), "us_per_step_two_calls": round(ms * 1e3, 3),
            "vectors_per_step": 2 * n, "vectors_per_s": round(2 * n / ms_pair * 1e3, 1),
            "workload": "one new token per (sequence, KV head): batch 64 x 8 KV heads, d=128, K 3+1-bit prod and "
                        "V 3-bit MSE appended into a 4096-token-per-head cache (one tq_append_kv_pair call per step; "
                        "two tq_append_kv calls beside it)"}


def decode_step(steps=100):
    """One decode step per call: append every (sequence, KV head)'s new key and value, then attend.

    tq_decode_step (the appends inside the decode's query-transform launch)
    against the two-call sequence (tq_append_kv_pair, then tq_decode_attn)
    and against the decode alone, each as a graph of `steps` calls whose
    lengths grow by one token per call. d = 128, K 3+1-bit prod (S R folded),
    V 3-bit MSE, bf16 rows; the caches stay resident in the last-level cache
    where they fit (the batch-1 one does), so the launch costs dominate there.
    """
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    res = {}
    for name, B, Hq, Hkv, T in (("batch 1 x 32768 tokens", 1, 32, 8, 32768),
                                ("batch 64 x 4096 tokens", 64, 32, 8, 4096)):
        d = 128
        n = B * Hkv * T
        Rk_t, Sk_t = dev(synth.haar_orthogonal(d, 8)), dev(synth.gaussian_matrix(d, d, 8))
        Rv_t = dev(synth.haar_orthogonal(d, 8, synth.STREAM_R_V))
        qk = tq.tq_quantizer_init(d, 3, tq.TQ_PROD, Rk_t, Sk_t)
        SR = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
        tq.tq_quantizer_fold(qk, SR)
        qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
        kp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, n) // 4, dtype=torch.int32,
                         device="cuda")
        vp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n) // 4, dtype=torch.int32,
                         device="cuda")
        kn, kr, vn = (torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(3))
        X = sdev.kv_with_outliers(B, Hkv, T, d, 4, 10.0, seed=8, stream=41).view(n, d)
        tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, X, n, d, kp, kn, kr)
        X = sdev.kv_with_outliers(B, Hkv, T, d, 4, 10.0, seed=8, stream=42).view(n, d)
        tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, X, n, d, vp, vn)
        del X
        kd = tq.make_desc([tq.make_group(qk, 0, kp, kn, kr, T)])
        vd = tq.make_desc([tq.make_group(qv, 0, vp, vn, None, T)])
        gen = sdev.generator(8, 43)
        k_new = torch.randn((B * Hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
        v_new = torch.randn((B * Hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
        q_t = torch.randn((B, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        wsb = tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, T)
        ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
        scale = 1.0 / math.sqrt(d)
        start = T - steps - 1
        lens = [torch.full((B,), start + 1 + i, dtype=torch.int32, device="cuda") for i in range(steps)]
        base = torch.arange(B * Hkv, device="cuda", dtype=torch.int64) * T
        rows = [base + (start + i) for i in range(steps)]

        def fused(i):
            tq.tq_decode_step(kd, vd, k_new, v_new, tq.TQ_BF16, q_t, tq.TQ_BF16, B, Hq, Hkv, T, lens[i % steps],
                              scale, out, None, ws, wsb)

        def two_calls(i):
            tq.tq_append_kv_pair(qk, qv, tq.TQ_BF16, k_new, v_new, B * Hkv, d, d, rows[i % steps], n, kp, kn, kr, vp,
                                 vn)
            tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T, lens[i % steps], scale, out, None, ws, wsb)

        def decode_only(i):
            tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T, lens[i % steps], scale, out, None, ws, wsb)

        r = {}
        for label, fn in (("tq_decode_step_us", fused), ("append_pair_then_decode_us", two_calls),
                          ("decode_alone_us", decode_only)):
            ms, _, _ = graph_ms(fn, steps)
            r[label] = round(ms * 1e3, 3)
        r["append_cost_in_step_us"] = round(r["tq_decode_step_us"] - r["decode_alone_us"], 3)
        r["append_cost_two_calls_us"] = round(r["append_pair_then_decode_us"] - r["decode_alone_us"], 3)
        res[name] = r
        del kp, vp, kn, kr, vn
        torch.cuda.empty_cache()
    res["workload"] = ("one new token per (sequence, KV head) appended and attended per step, 32 q / 8 KV heads, "
                       "d=128, K 3+1-bit prod (S R folded), V 3-bit MSE; graphs of 100 steps")
    return res


NIAH_KEYS = [("3+1 prod", 3, True), ("4 MSE-only", 4, False), ("2+1 prod", 2, True), ("3 MSE-only", 3, False),
             ("1+1 prod", 1, True)]


def niah_proxy(lengths=(1024, 4096, 16384), cosines=(0.4, 0.5), B=8):
    """Needle-in-a-haystack proxy: is the needle still the top-scoring token?

    Per (sequence, KV head) one needle key is planted at a seeded position
    among keys of the headline law (bf16 N(0, 1), 4 channels x10): its
    direction has cosine `c` with the group's first query head (the rest a
    random direction orthogonal to it) and its norm is the median key norm of
    that head. The needle's parameters are unstated in the pages, so this
    reproduces the trend only. Reported per (length, cosine, key allocation):
    the fraction of (sequence, KV head) trials whose exact fp64 score argmax
    is the needle, and the fraction whose libtq score estimate argmax is.
    """
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    Hq, Hkv, d = 32, 8, 128
    G = Hq // Hkv
    Rk_t = dev(synth.haar_orthogonal(d, 7))
    Sk_t = dev(synth.gaussian_matrix(d, d, 7))
    Rv_t = dev(synth.haar_orthogonal(d, 7, synth.STREAM_R_V))
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
    quants = []
    for name, kb, kprod in NIAH_KEYS:
        q = tq.tq_quantizer_init(d, kb, tq.TQ_PROD if kprod else tq.TQ_MSE, Rk_t, Sk_t if kprod else None)
        SR = None
        if kprod:
            SR = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
            tq.tq_quantizer_fold(q, SR)
        quants.append((name, kb, kprod, q, SR))
    rows = []
    for L in lengths:
        n = B * Hkv * L
        V = sdev.kv_with_outliers(B, Hkv, L, d, 4, 10.0, seed=L, stream=21)
        vp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n) // 4, dtype=torch.int32,
                         device="cuda")
        vn = torch.empty(n, dtype=torch.int16, device="cuda")
        tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, V.view(n, d), n, d, vp, vn)
        vd = tq.make_desc([tq.make_group(qv, 0, vp, vn, None, L)])
        gen = sdev.generator(L, 22)
        qry = torch.randn((B, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
        for c in cosines:
            K = sdev.kv_with_outliers(B, Hkv, L, d, 4, 10.0, seed=L, stream=20)
            pos = torch.randint(0, L, (B, Hkv), generator=gen, device="cuda")
            qh = qry[:, ::G].float()  # [B, Hkv, d]: each group's first query head
            qhat = qh / qh.norm(dim=-1, keepdim=True)
            rnd = torch.randn((B, Hkv, d), generator=gen, device="cuda")
            rnd -= (rnd * qhat).sum(-1, keepdim=True) * qhat
            rnd /= rnd.norm(dim=-1, keepdim=True)
            knorm = K.float().norm(dim=-1).median(dim=-1).values  # [B, Hkv]
            needle = (c * qhat + math.sqrt(1 - c * c) * rnd) * knorm[..., None]
            bi = torch.arange(B, device="cuda")[:, None].expand(B, Hkv)
            gi = torch.arange(Hkv, device="cuda")[None, :].expand(B, Hkv)
            K[bi, gi, pos] = needle.to(torch.bfloat16)
            ex = torch.matmul(K.double(), qh.double()[..., None])[..., 0]  # [B, Hkv, L] exact scores
            exact_hit = (ex.argmax(dim=-1) == pos).float().mean().item()
            for name, kb, kprod, q, _ in quants:
                kp = torch.empty(tq.tq_packed_bytes(d, kb, tq.TQ_PROD if kprod else tq.TQ_MSE, tq.TQ_LAYOUT_KEYS, n)
                                 // 4, dtype=torch.int32, device="cuda")
                kn = torch.empty(n, dtype=torch.int16, device="cuda")
                kr = torch.empty(n, dtype=torch.int16, device="cuda") if kprod else None
                tq.tq_quantize_kv(q, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, K.view(n, d), n, d, kp, kn, kr)
                kd = tq.make_desc([tq.make_group(q, 0, kp, kn, kr, L)])
                wsb = tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, L)
                ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
                out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
                sc = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
                tq.tq_decode_attn(kd, vd, qry, tq.TQ_BF16, B, Hq, Hkv, L, None, 1 / math.sqrt(d), out, sc, ws, wsb)
                torch.cuda.synchronize()
                hit = (sc[:, ::G].argmax(dim=-1) == pos).float().mean().item()
                rows.append({"seq_len": L, "needle_cosine": c, "keys": name, "exact_top1": round(exact_hit, 4),
                             "libtq_top1": round(hit, 4)})
                log(f"niah proxy {rows[-1]}")
            del K, ex
        del V, vp, vn
        torch.cuda.empty_cache()
    return {"workload": f"{B} sequences x 8 KV heads per length, 32 q heads, d=128, values 3-bit MSE; one needle "
                        "per (sequence, KV head) at a seeded position, scored against the group's first query head",
            "rows": rows}


def paged_decode(steps=20):
    """Decode from a paged cache against the same cache stored contiguously.

    Batch 16 x 32768 tokens, 32 q / 8 KV heads, d = 128, K 3+1-bit prod and
    V 3-bit MSE (the single-layer law). The pool's 4096-token blocks are
    copies of the contiguous cache's block slices scattered over a shuffled
    pool, so the two decodes read the same codes and differ only in
    addressing and split lengths. Separately, the same vectors are quantised
    by the append path (the general kernel) to report how often it decides a
    code bit differently from the bulk matrix-core quantiser.
    """
    import numpy as np
    import torch

    import decode_tq_quantize_amd as tq
    import synth
    from synth import device as sdev

    B, Hq, Hkv, T, d, bt = 16, 32, 8, 32768, 128, 4096
    n = B * Hkv * T
    nbs = T // bt
    Rk_t, Sk_t = dev(synth.haar_orthogonal(d, 6)), dev(synth.gaussian_matrix(d, d, 6))
    Rv_t = dev(synth.haar_orthogonal(d, 6, synth.STREAM_R_V))
    qk = tq.tq_quantizer_init(d, 3, tq.TQ_PROD, Rk_t, Sk_t)
    SR = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
    tq.tq_quantizer_fold(qk, SR)
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rv_t)
    perm = torch.from_numpy(synth.rng(6, 7).permutation(B * nbs).astype(np.int64)).cuda()
    table = perm.view(B, nbs).to(torch.int32).contiguous()
    # block (b, g, j) of the contiguous cache -> pool block table[b, j] * Hkv + g
    src_blk = torch.arange(B * Hkv * nbs, device="cuda")
    b_i = src_blk // (Hkv * nbs)
    g_i = (src_blk // nbs) % Hkv
    j_i = src_blk % nbs
    dst_blk = table.long()[b_i, j_i] * Hkv + g_i
    keep, descs, flips = [], {}, {}
    identity = torch.arange(n, device="cuda", dtype=torch.int64)
    for name, q, lay, var, st in (("k", qk, tq.TQ_LAYOUT_KEYS, tq.TQ_PROD, 1),
                                  ("v", qv, tq.TQ_LAYOUT_VALUES, tq.TQ_MSE, 2)):
        X = sdev.kv_with_outliers(B, Hkv, T, d, 4, 10.0, seed=6, stream=st).view(n, d)
        nb = tq.tq_packed_bytes(d, 3, var, lay, n)
        pk = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
        nr = torch.empty(n, dtype=torch.int16, device="cuda")
        rr = torch.empty(n, dtype=torch.int16, device="cuda") if var == tq.TQ_PROD else None
        tq.tq_quantize_kv(q, lay, tq.TQ_BF16, X, n, d, pk, nr, rr)
        # the pool: each block slice copied to its shuffled place (blocks are
        # whole tiles of both layouts, so a block is one contiguous range)
        pp = torch.zeros_like(pk)
        pp.view(B * Hkv * nbs, -1)[dst_blk] = pk.view(B * Hkv * nbs, -1)[src_blk]
        pn = torch.zeros_like(nr)
        pn.view(B * Hkv * nbs, bt)[dst_blk] = nr.view(B * Hkv * nbs, bt)[src_blk]
        pr = None
        if rr is not None:
            pr = torch.zeros_like(rr)
            pr.view(B * Hkv * nbs, bt)[dst_blk] = rr.view(B * Hkv * nbs, bt)[src_blk]
        # the append path's codes for the same vectors, row for row
        ap = torch.zeros_like(pk)
        an = torch.zeros_like(nr)
        ar = torch.zeros_like(rr) if rr is not None else None
        tq.tq_append_kv(q, lay, tq.TQ_BF16, X, n, d, identity, n, ap, an, ar)
        torch.cuda.synchronize()
        xor = torch.bitwise_xor(ap, pk)
        bits_diff = int(sum(int(((xor >> s) & 1).sum()) for s in range(32)))
        flips[name] = {"code_and_sign_bits_differing": bits_diff, "bits": nb * 8,
                       "rate": bits_diff / (nb * 8),
                       "norms_differing": int((an != nr).sum()),
                       "residual_norms_differing": int((ar != rr).sum()) if rr is not None else 0}
        del X, ap, an, ar, xor
        keep += [pk, pp, nr, pn, rr, pr]
        descs[name] = (tq.make_desc([tq.make_group(q, 0, pk, nr, rr, T)]),
                       tq.make_desc([tq.make_group(q, 0, pp, pn, pr, bt)]))
    q_t = torch.randn((B, Hq, d), generator=sdev.generator(6, 8), device="cuda").to(torch.bfloat16)
    out_c = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    out_p = torch.empty_like(out_c)
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    wsc = tq.tq_decode_workspace_bytes(descs["k"][0], descs["v"][0], B, Hq, Hkv, T)
    wsp = tq.tq_decode_paged_workspace_bytes(descs["k"][1], descs["v"][1], B, Hq, Hkv, T, bt)
    ws_c = torch.empty(wsc // 4 + 4, dtype=torch.float32, device="cuda")
    ws_p = torch.empty(wsp // 4 + 4, dtype=torch.float32, device="cuda")

    def contiguous(i=0):
        tq.tq_decode_attn(descs["k"][0], descs["v"][0], q_t, tq.TQ_BF16, B, Hq, Hkv, T, lens, 1 / math.sqrt(d),
                          out_c, None, ws_c, wsc)

    def paged(i=0):
        tq.tq_decode_attn_paged(descs["k"][1], descs["v"][1], q_t, tq.TQ_BF16, B, Hq, Hkv, T, lens, table, nbs, bt,
                                B * nbs, 1 / math.sqrt(d), out_p, None, ws_p, wsp)

    res = {}
    for name, fn in (("contiguous", contiguous), ("paged", paged)):
        res[name], _, _ = graph_ms(fn, steps)
    diff = (out_p - out_c).double().norm(dim=-1) / out_c.double().norm(dim=-1)
    bytes_ = n * 118 + B * Hq * d * 6
    return {"contiguous_ms": round(res["contiguous"], 4), "paged_ms": round(res["paged"], 4),
            "paged_gbs": round(bytes_ / res["paged"] / 1e6, 1),
            "paged_hbm_frac": round(bytes_ / res["paged"] / 1e6 / HBM_PEAK_GBS, 4),
            "paged_vs_contiguous_output_rel_diff_max": float(diff.max()),
            "append_vs_bulk_quantiser": flips,
            "workload": "batch 16 x 32768 tokens, 32 q / 8 KV heads, d=128, K 3+1-bit prod, V 3-bit MSE; the paged "
                        "copy is the contiguous cache's 4096-token blocks over a shuffled pool"}


def run_extra(extras, name, fn):
    try:
        extras[name] = fn()
    except Exception as e:  # an extra that fails is reported, not hidden
        extras[name] = {"error": repr(e)}
    log(f"{name}: {extras[name]}")


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X and no multi-GPU job is launched; "
              "pass --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_tq_quantize_amd as tq

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    tq.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    head = longctx_decode(args)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_longctx(head["oracle"], head["call_bytes"])
        log(f"cpu baseline: {cpu}")
    extras = {"longctx_decode": head["extras"]}
    only = set(x for x in args.only.split(",") if x)
    want = (lambda key: not args.no_extras and (not only or key in only))
    with_cpu = not args.no_cpu
    single = None
    if want("single") or want("bits"):
        try:
            single = single_layer_decode(cpu=with_cpu)
            extras["single_layer_decode"] = {k: v for k, v in single.items() if k != "oracle_inputs"}
        except Exception as e:
            extras["single_layer_decode"] = {"error": repr(e)}
    if want("tiny"):
        run_extra(extras, "tiny_score_matrix", lambda: tiny_score_matrix(cpu=with_cpu))
    if want("quantize"):
        run_extra(extras, "quantize_prefill", lambda: quantize_prefill(cpu=with_cpu))
    if want("search"):
        run_extra(extras, "vector_search", lambda: vector_search(cpu=with_cpu))
    if want("paged"):
        run_extra(extras, "paged_decode", paged_decode)
    if want("append"):
        run_extra(extras, "append_step", append_step)
    if want("step"):
        run_extra(extras, "decode_step", decode_step)
    if want("niah"):
        run_extra(extras, "niah_proxy", niah_proxy)
    if want("bits") and single is not None and "oracle_inputs" in single:
        run_extra(extras, "bit_allocations", lambda: bit_allocations(single["oracle_inputs"]))
    traffic = measured_traffic("longctx_decode")
    line = {
        "metric": METRIC,
        "value": round(head["call_bytes"] / (head["per_call_ms"] * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["per_call_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DECODE_DTYPE,
        "data": "synthetic",
        "config": {"workload": "long-context batched decode attention from compressed KV: batch 64 x 131072 tokens, "
                               "32 q / 8 KV heads, head_dim 128, one layer, 2.5 bits per channel",
                   "batch": LC["B"], "seq_len": LC["T"], "q_heads": LC["Hq"], "kv_heads": LC["Hkv"],
                   "head_dim": LC["d"],
                   "keys": "TurboQuant_prod: 32 outlier channels 2+1 bits, 96 channels 1+1 bits",
                   "values": "TurboQuant_mse: 32 outlier channels 3 bits, 96 channels 2 bits",
                   "bytes_per_token_head": LC_BYTES_PER_TOKEN_HEAD, "parallelism": "none (1 GPU)"},
        "roofline": roofline_block(head["kv_bytes"], head["dk_ms"], head["call_bytes"], head["per_call_ms"], traffic,
                                   "decode_kernel (compressed-cache scores, softmax and value sums; HIP events around "
                                   "a graph of its launches alone, chained)"),
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
