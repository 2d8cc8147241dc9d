#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one call of each entry point of the hot path on its workload, inputs
resident in HBM:
  attn_fwd           B=1 H=32 N=8192 d=128 bf16 causal          (headline, TFLOP/s)
  attn_fwd_varlen    16 sequences, lengths U[128,4096], H=32 d=128 bf16 causal
  attn_decode_paged  64 sequences, context U[512,8192], 16-token pages, H=32 d=128 bf16
                     (headline, HBM GB/s)
After the timed steps, the further entry points are timed the same way in a loop of
their own (reported per entry point, not part of ms_per_step):
  attn_fwd           B=1 H=1 N=256 d=64 fp32 non-causal             (time only)
  attn_fwd           B=4 H=16 N=2048 d=128 bf16 non-causal          (TFLOP/s)
  attn_decode_paged  the same lengths with 16 query heads on 8 KV heads (grouped-query)
  attn_store_kvcache the varlen batch's 34069 new K/V rows written into 16-token pages
  attn_fwd_varlen    paged prefill: the second half of each of those sequences as new
                     causal rows over its whole context, read through the block table
  attn_bwd           dQ, dK, dV of the dense causal forward (by recomputation)
  attn_bwd_varlen    dQ, dK, dV of the varlen forward

W untimed warm-up steps, then K timed steps; every kernel call is bracketed by HIP
events on the stream it runs on.  Prints ONE JSON line.  `value` is the dense
forward's algorithmic TFLOP/s (admissible query-key pairs x 4d flops / average
launch time).  Every leg reports the mean, median and minimum of its launches and
their count.  The fp64 CPU oracle is timed on a bounded sample of each of the five
workloads as `cpu_baseline` (the headline figure is the causal dense one).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "attn fwd TFLOP/s + %MFMA peak (N=8192,d=128 bf16); paged decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

# HBM bytes per launch of the dense forward kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# (KiB per dispatch), scaled by what the same counters read for a 512 MiB device copy
# (FETCH_SIZE reads half of the bytes moved: x2; WRITE_SIZE x1), per workload.  Valid
# only for the kernel source they were taken on (sha256 prefix of attn_fwd.hip followed
# by the attn_tile.h and attn_internal.h it includes); reported as null otherwise.
FWD_COUNTERS = {"source_sha256_16": "7d972f05332f4deb", "fetch_scale": 2.0, "write_scale": 1.0,
                "c3": {"fetch_kib": 130930.9375, "write_kib": 66560.0},
                "c2": {"fetch_kib": 49280.5, "write_kib": 33280.0}}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops_causal(H: int, N: int, d: int, B: int = 1) -> float:
    """4*d flops per admissible (query, key) pair; causal admits N(N+1)/2 pairs."""
    return 4.0 * d * B * H * N * (N + 1) / 2


def varlen_flops(lens, H: int, d: int) -> float:
    L = np.asarray(lens, dtype=np.float64)
    return float(np.sum(2.0 * d * H * L * (L + 1)))


def decode_bytes(ctx, B: int, H: int, d: int, page: int, H_kv: int | None = None) -> int:
    """Ideal HBM traffic: each context token's K and V once (H_kv heads), q read, O and
    lse written (H heads), the used block-table entries and the context lengths."""
    H_kv = H if H_kv is None else H_kv
    c = np.asarray(ctx, dtype=np.int64)
    return int(c.sum() * H_kv * d * 2 * 2 + B * H * d * 2 * 2 + B * H * 4 + ((c + page - 1) // page).sum() * 4 + B * 4)


def fwd_bytes(B: int, H: int, N: int, d: int) -> int:
    return B * H * (4 * N * d * 2 + 4 * N)


def fwd_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "attn_tile.h", "attn_internal.h"):
        with open(os.path.join(ROOT, "exact_attention_attn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fwd_traffic_bytes(workload: str):
    """Counter-measured HBM bytes per dense forward launch on ``workload``, or None if
    the kernel source changed since the counters were taken (or none were taken)."""
    c = FWD_COUNTERS
    if fwd_source_hash() != c["source_sha256_16"] or c.get(workload) is None:
        return None
    w = c[workload]
    return (w["fetch_kib"] * c["fetch_scale"] + w["write_kib"] * c["write_scale"]) * 1024.0


def dev(x: np.ndarray):
    """Host array -> torch GPU tensor (uint16 arrays are bf16 bit patterns)."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def stats(ms: np.ndarray) -> dict:
    """Mean, median, minimum (ms) and count of one leg's launch times."""
    return {"ms": float(ms.mean()), "ms_median": float(np.median(ms)), "ms_min": float(ms.min()),
            "launches": int(ms.size)}


def host_cores() -> dict:
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = None
    return {"os_cpu_count": os.cpu_count(), "sched_getaffinity": aff, "blas_threads": blas}


def cpu_baseline(ws: dict, gpu_ms: dict, budget_s: dict) -> dict:
    """Time the fp64 oracle (as it stands, untuned) on each workload in ``ws``: whole
    heads (or whole (sequence, head) pairs) until that workload's time budget is used.
    Each entry reports the sample, its wall time, the oracle's rate on the algorithmic
    work it covered (flops, or bytes for decode) and the GPU/oracle speed ratio on the
    same rate.  The headline value is the causal dense workload's TFLOP/s."""
    import oracle
    out = {}

    def timed(items, fn):
        t0 = time.perf_counter()
        done = []
        for it in items:
            fn(it)
            done.append(it)
            if time.perf_counter() - t0 > budget_s[name]:
                break
        return done, time.perf_counter() - t0

    for name, w in ws.items():
        if name == "c1":
            reps, dt = timed(range(20), lambda _: oracle.attention_rows(w.q[0, 0], w.k[0, 0], w.v[0, 0], w.scale,
                                                                        w.causal))
            fl = len(reps) * 4.0 * w.d * w.N * w.N
            gfl = 4.0 * w.d * w.N * w.N
            e = {"sample": f"the whole workload, {len(reps)} times", "unit": "TFLOP/s"}
        elif name in ("c2", "c3"):
            pairs = [(b, h) for h in range(w.H) for b in range(w.B)]
            done, dt = timed(pairs, lambda bh: oracle.attention_rows(w.q[bh[0], bh[1]], w.k[bh[0], bh[1]],
                                                                     w.v[bh[0], bh[1]], w.scale, w.causal))
            per = fwd_flops_causal(1, w.N, w.d) if w.causal else 4.0 * w.d * w.N * w.N
            fl, gfl = len(done) * per, len(pairs) * per
            e = {"sample": f"{len(done)} of {len(pairs)} (batch, head) pairs", "unit": "TFLOP/s"}
        elif name == "c4":
            lens = np.diff(w.cu_q)
            items = [(h, s) for h in range(32) for s in range(len(lens))]
            cu = w.cu_q
            done, dt = timed(items, lambda hs: oracle.attention_rows(
                w.q[cu[hs[1]]:cu[hs[1] + 1], hs[0]], w.k[cu[hs[1]]:cu[hs[1] + 1], hs[0]],
                w.v[cu[hs[1]]:cu[hs[1] + 1], hs[0]], w.scale, True))
            fl = float(sum(2.0 * w.d * lens[s] * (lens[s] + 1.0) for _, s in done))
            gfl = varlen_flops(lens, 32, w.d)
            e = {"sample": f"{len(done)} of {len(items)} (sequence, head) pairs", "unit": "TFLOP/s"}
        else:  # c5: decode, rate in bytes
            items = list(range(32))
            done, dt = timed(items, lambda h: oracle.attention_decode_paged(
                w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale, heads=[h]))
            fl = decode_bytes(w.context_lens, 64, len(done), 128, 16)
            gfl = decode_bytes(w.context_lens, 64, 32, 128, 16)
            e = {"sample": f"{len(done)} of 32 heads, all 64 sequences", "unit": "GB/s"}
        div = 1e12 if e["unit"] == "TFLOP/s" else 1e9
        e["value"] = fl / dt / div
        e["wall_s"] = dt
        if name in gpu_ms:
            gpu_rate = gfl / (gpu_ms[name] / 1e3) / div
            e["gpu_value"] = gpu_rate
            e["gpu_over_oracle"] = gpu_rate / e["value"]
        out[name] = e
        log(f"[bench] oracle {name}: {e['value']:.4g} {e['unit']} on {e['sample']} ({dt:.1f} s)")
    c3 = out["c3"]
    cores = host_cores()
    return {"value": c3["value"], "unit": "TFLOP/s", "cores": cores["blas_threads"] or cores["sched_getaffinity"],
            "kind": "oracle", "sample": f"causal B=1 H=32 N=8192 d=128: {c3['sample']} (fp64 NumPy, "
                                        f"{c3['wall_s']:.1f} s); the other workloads under 'configs'",
            "host": cores, "configs": out}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fwd", "varlen", "decode", "c1", "c2", "decode_gqa", "store_kvcache",
                                       "prefill_paged", "bwd", "bwd_varlen"],
                    default=None,
                    help="time one entry point only (profiling aid); the JSON line is still printed")
    ap.add_argument("--gqa-batch", type=int, default=64,
                    help="sequences of the grouped-query decode leg (64: the workload of the JSON line; more: "
                         "the same length distribution on a larger batch, to separate launch ramp from steady state)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not implemented.", file=sys.stderr)
        return 2

    import torch

    import exact_attention_attn_amd as attn
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    attn.load()
    dev_name = torch.cuda.get_device_name(0)

    # legs to run and the workloads they need (only those are generated)
    step_names = ["fwd", "varlen", "decode"]
    extra_names = ["c1", "c2", "decode_gqa", "store_kvcache", "prefill_paged", "bwd", "bwd_varlen"]
    if args.only:
        step_names = [n for n in step_names if n == args.only]
        extra_names = [n for n in extra_names if n == args.only]
    need = set(step_names + extra_names)
    with_cpu = not args.no_cpu_baseline and "fwd" in need
    if with_cpu:
        need |= {"c1", "c2", "fwd", "varlen", "decode"}
    if "bwd" in need:
        need.add("fwd")
    if "bwd_varlen" in need:
        need.add("varlen")

    t = time.perf_counter()
    if "c1" in need:
        w1 = synth.workload("c1")
        q1, k1, v1 = dev(w1.q), dev(w1.k), dev(w1.v)
        o1 = torch.empty_like(q1)
        l1 = torch.empty((1, 1, w1.N), dtype=torch.float32, device="cuda")
    if "c2" in need:
        w2 = synth.workload("c2")
        q2, k2, v2 = dev(w2.q), dev(w2.k), dev(w2.v)
        o2 = torch.empty_like(q2)
        l2 = torch.empty((w2.B, w2.H, w2.N), dtype=torch.float32, device="cuda")
    if "fwd" in need:
        w3 = synth.workload("c3")
        q3, k3, v3 = dev(w3.q), dev(w3.k), dev(w3.v)
        o3 = torch.empty_like(q3)
        l3 = torch.empty((1, 32, 8192), dtype=torch.float32, device="cuda")
    log(f"[bench] dense workloads ready ({time.perf_counter() - t:.1f} s)")

    if "varlen" in need:
        w4 = synth.workload("c4")
        q4, k4, v4 = dev(w4.q), dev(w4.k), dev(w4.v)
        cq4, ck4 = dev(w4.cu_q), dev(w4.cu_k)
        o4 = torch.empty_like(q4)
        l4 = torch.empty((q4.shape[0], 32), dtype=torch.float32, device="cuda")
        log(f"[bench] varlen workload ready ({time.perf_counter() - t:.1f} s)")

    if "decode" in need:
        w5 = synth.workload("c5")
        q5, kc5, vc5 = dev(w5.q), dev(w5.k_cache), dev(w5.v_cache)
        bt5, cl5 = dev(w5.block_table), dev(w5.context_lens)
        maxctx5 = int(w5.context_lens.max())
        ws5 = torch.empty(attn.attn_decode_paged_workspace_size(64, 32, 128, maxctx5, 16), dtype=torch.uint8,
                          device="cuda")
        o5 = torch.empty_like(q5)
        l5 = torch.empty((64, 32), dtype=torch.float32, device="cuda")
        # (the host copies stay: the oracle's timed sample reads them)
        log(f"[bench] decode workload ready ({time.perf_counter() - t:.1f} s)")

    if "decode_gqa" in need:
        w6 = synth.workload("gqa_decode") if args.gqa_batch == 64 else \
            synth.paged(args.gqa_batch, 16, 128, 512, 8192, 16, seed=0, H_kv=8)
        q6, kc6, vc6 = dev(w6.q), dev(w6.k_cache), dev(w6.v_cache)
        bt6, cl6 = dev(w6.block_table), dev(w6.context_lens)
        maxctx6 = int(w6.context_lens.max())
        ws6 = torch.empty(attn.attn_decode_paged_workspace_size(w6.B, 16, 128, maxctx6, 16), dtype=torch.uint8,
                          device="cuda")
        o6 = torch.empty_like(q6)
        l6 = torch.empty((w6.B, 16), dtype=torch.float32, device="cuda")
        w6.k_cache = w6.v_cache = None
        log(f"[bench] grouped-query decode workload ready ({time.perf_counter() - t:.1f} s)")

    if "prefill_paged" in need:
        w8 = synth.workload("prefill_paged")
        q8, kc8, vc8 = dev(w8.q), dev(w8.k_cache), dev(w8.v_cache)
        cq8, ck8, bt8 = dev(w8.cu_q), dev(w8.cu_k), dev(w8.block_table)
        o8 = torch.empty_like(q8)
        l8 = torch.empty((q8.shape[0], 32), dtype=torch.float32, device="cuda")
        w8.k_cache = w8.v_cache = None
        log(f"[bench] paged prefill workload ready ({time.perf_counter() - t:.1f} s)")

    if "bwd" in need:
        do3 = dev(synth.normal(0, synth.T_DO, (1, 32, 8192, 128), True))
        dq3, dk3, dv3 = torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3)
        wsb = torch.empty(attn.attn_bwd_workspace_size(1, 32, 8192), dtype=torch.uint8, device="cuda")
        log(f"[bench] backward workload ready ({time.perf_counter() - t:.1f} s)")

    if "bwd_varlen" in need:
        do4 = dev(synth.normal(0, synth.T_DO, tuple(w4.q.shape), True))
        dq4, dk4, dv4 = torch.empty_like(q4), torch.empty_like(k4), torch.empty_like(v4)
        wsb4 = torch.empty(attn.attn_bwd_varlen_workspace_size(q4.shape[0], 32), dtype=torch.uint8, device="cuda")
        log(f"[bench] varlen backward workload ready ({time.perf_counter() - t:.1f} s)")

    if "store_kvcache" in need:
        w7 = synth.workload("store_prefill")
        k7, v7, kc7, vc7 = dev(w7.k), dev(w7.v), dev(w7.k_cache), dev(w7.v_cache)
        sl7 = torch.from_numpy(w7.slot_mapping).cuda()
        log(f"[bench] store_kvcache workload ready ({time.perf_counter() - t:.1f} s)")

    def run_fwd():
        attn.attn_fwd(q3, k3, v3, scale=w3.scale, causal=True, out=o3, lse=l3)

    def run_c1():
        attn.attn_fwd(q1, k1, v1, scale=w1.scale, causal=False, out=o1, lse=l1)

    def run_c2():
        attn.attn_fwd(q2, k2, v2, scale=w2.scale, causal=False, out=o2, lse=l2)

    def run_varlen():
        attn.attn_fwd_varlen(q4, k4, v4, cq4, ck4, w4.max_q, w4.max_k, scale=w4.scale, causal=True, out=o4, lse=l4)

    def run_decode():
        attn.attn_decode_paged(q5, kc5, vc5, bt5, cl5, maxctx5, scale=w5.scale, workspace=ws5, out=o5, lse=l5)

    def run_decode_gqa():
        attn.attn_decode_paged(q6, kc6, vc6, bt6, cl6, maxctx6, scale=w6.scale, workspace=ws6, out=o6, lse=l6)

    def run_store():
        attn.attn_store_kvcache(k7, v7, kc7, vc7, sl7)

    def run_bwd():
        attn.attn_bwd(q3, k3, v3, o3, l3, do3, scale=w3.scale, causal=True, dq=dq3, dk=dk3, dv=dv3, workspace=wsb)

    def run_bwd_varlen():
        attn.attn_bwd_varlen(q4, k4, v4, o4, l4, do4, cq4, ck4, w4.max_q, w4.max_k, scale=w4.scale, causal=True,
                             dq=dq4, dk=dk4, dv=dv4, workspace=wsb4)

    def run_prefill_paged():
        attn.attn_fwd_varlen(q8, kc8, vc8, cq8, ck8, w8.max_q, w8.max_k, scale=w8.scale, causal=True,
                             out=o8, lse=l8, block_table=bt8)

    # The timed step is the hot path proper: the dense forward, the varlen forward and
    # paged decode.  The further entry points (grouped-query decode, store_kvcache, paged
    # prefill, both backward passes) are timed after it, in a loop of their own of the
    # same length, so that their heat does not lower the clock under the step's legs.
    fns = {"fwd": run_fwd, "varlen": run_varlen, "decode": run_decode, "c1": run_c1, "c2": run_c2,
           "decode_gqa": run_decode_gqa, "store_kvcache": run_store, "prefill_paged": run_prefill_paged,
           "bwd": run_bwd, "bwd_varlen": run_bwd_varlen}
    parts = [(n, fns[n]) for n in step_names]
    extra = [(n, fns[n]) for n in extra_names]

    def timed_loop(legs):
        """W warm-up rounds, then K timed rounds of `legs`, each call bracketed by HIP
        events on the current stream; returns the per-leg times and the loop's time."""
        for _ in range(args.warmup):
            for _, fn in legs:
                fn()
        torch.cuda.synchronize()
        ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(args.steps)] for name, _ in legs}
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            for name, fn in legs:
                a, b = ev[name][i]
                a.record()
                fn()
                b.record()
        end.record()
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        times = {name: np.array([a.elapsed_time(b) for a, b in ev[name]]) for name, _ in legs}
        return times, start.elapsed_time(end), wall_s

    ms, ms_total, wall = timed_loop(parts) if parts else ({}, 0.0, 0.0)
    if extra:
        ms_extra, _, _ = timed_loop(extra)
        ms.update(ms_extra)
    for name in ms:
        log(f"[bench] {name}: mean {ms[name].mean():.4f} ms  median {np.median(ms[name]):.4f}  min {ms[name].min():.4f}")

    fl3 = fwd_flops_causal(32, 8192, 128)
    fl2 = 4.0 * 128 * 4 * 16 * 2048 * 2048
    fl1 = 4.0 * 64 * 256 * 256
    fl4 = varlen_flops(w4.lens_q, 32, 128) if "varlen" in need else None
    by5 = decode_bytes(w5.context_lens, 64, 32, 128, 16) if "decode" in need else None
    res = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_total / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "causal attention forward B=1 H=32 N=8192 d=128 bf16 (fp32 accumulate)",
                      "step": [p[0] for p in parts], "also_timed": [p[0] for p in extra], "device": dev_name,
                      "fwd_source_sha256_16": fwd_source_hash()}}

    def rate(name, work, unit, peak):
        """Stats of leg ``name`` plus its rate on ``work`` (flops or bytes per launch) and
        the fraction of ``peak`` (None: no roofline claim)."""
        e = stats(ms[name])
        div = 1e12 if unit == "TFLOP/s" else 1e9
        key = "tflops" if unit == "TFLOP/s" else "GB/s"
        e[key] = work / (e["ms"] / 1e3) / div
        if peak is not None:
            e["peak"] = peak
            e["frac"] = e[key] / peak
        return e

    if "fwd" in ms:
        e = rate("fwd", fl3, "TFLOP/s", PEAK_BF16_TFLOPS)
        res["value"] = e["tflops"]
        res["fwd"] = e
        res["roofline"] = {"bound": "mfma", "achieved": e["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": e["frac"], "traffic": fwd_traffic_bytes("c3"),
                           "kernel": "fwd_bf16_kernel<128, 4, 64, 2, true, false, false>", "flops_per_launch": fl3,
                           "algorithmic_bytes_per_launch": fwd_bytes(1, 32, 8192, 128)}
    else:
        res["value"] = None
    if "c1" in ms:
        res["c1"] = dict(workload="B=1 H=1 N=256 d=64 fp32 non-causal (fp32 VALU kernel; latency-bound, no "
                                  "roofline claim)", flops_per_launch=fl1, **rate("c1", fl1, "TFLOP/s", None))
    if "c2" in ms:
        res["c2"] = dict(workload="B=4 H=16 N=2048 d=128 bf16 non-causal", flops_per_launch=fl2,
                         kernel="fwd_bf16_kernel<128, 4, 64, 2, false, false, false>",
                         algorithmic_bytes_per_launch=fwd_bytes(4, 16, 2048, 128), traffic=fwd_traffic_bytes("c2"),
                         note="inputs (134 MB) fit the 256 MB last-level cache; compute-bound either way",
                         **rate("c2", fl2, "TFLOP/s", PEAK_BF16_TFLOPS))
    if "varlen" in ms:
        res["varlen"] = dict(workload="16 seqs len U[128,4096] (seed 0: 34069 tokens) H=32 d=128 bf16 causal",
                             flops_per_launch=fl4, **rate("varlen", fl4, "TFLOP/s", PEAK_BF16_TFLOPS))
    if "decode" in ms:
        res["decode"] = dict(workload="64 seqs ctx U[512,8192] (seed 0: 283360 tokens) 16-token pages H=32 d=128 bf16",
                             bytes_per_launch=by5, note="split kernel + combine kernel, both inside the timed launch",
                             **rate("decode", by5, "GB/s", PEAK_HBM_GBS))
    if "decode_gqa" in ms:
        by6 = decode_bytes(w6.context_lens, w6.B, 16, 128, 16, H_kv=8)
        res["decode_gqa"] = dict(workload=f"{w6.B} seqs ctx U[512,8192] (seed 0) 16-token pages H=16 H_kv=8 d=128 bf16",
                                 bytes_per_launch=by6, note="KV bytes counted once per KV head (grouped-query)",
                                 **rate("decode_gqa", by6, "GB/s", PEAK_HBM_GBS))
    if "bwd" in ms:
        flb = 2.5 * fl3   # five tile products per admissible pair (dV, dP, dQ, dK, and S)
        res["bwd"] = dict(workload="backward of the causal B=1 H=32 N=8192 d=128 forward (dQ, dK, dV)",
                          flops_per_launch=flb,
                          note="algorithmic flops 2.5x the forward's; the kernels recompute S and P twice",
                          **rate("bwd", flb, "TFLOP/s", PEAK_BF16_TFLOPS))
    if "bwd_varlen" in ms:
        flv = 2.5 * fl4   # of the varlen forward's
        res["bwd_varlen"] = dict(workload="backward of the 16-sequence varlen forward (dQ, dK, dV)",
                                 flops_per_launch=flv, **rate("bwd_varlen", flv, "TFLOP/s", PEAK_BF16_TFLOPS))
    if "prefill_paged" in ms:
        lq8, lk8 = w8.lens_q.astype(np.float64), w8.lens_k.astype(np.float64)
        fl8 = float(np.sum(4.0 * 128 * 32 * (lq8 * (lk8 - lq8) + lq8 * (lq8 + 1) / 2)))  # admissible pairs x 4d
        res["prefill_paged"] = dict(workload=f"16 seqs, {int(lq8.sum())} new causal rows over {int(lk8.sum())} "
                                             "context tokens in 16-token pages, H=32 d=128 bf16",
                                    flops_per_launch=fl8, **rate("prefill_paged", fl8, "TFLOP/s", PEAK_BF16_TFLOPS))
    if "store_kvcache" in ms:
        by7 = 4 * w7.T * w7.H_kv * w7.d * 2 + 8 * w7.T   # K and V read and written once, slots read
        res["store_kvcache"] = dict(workload=f"{w7.T} tokens H_kv=32 d=128 bf16 into 16-token pages",
                                    bytes_per_launch=by7, **rate("store_kvcache", by7, "GB/s", PEAK_HBM_GBS))
    res["wall_s_timed"] = wall
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 512 << 20
    if with_cpu:
        # bounded samples: about 25 s of oracle work in all on the host's cores
        gpu = {n: float(ms[m].mean()) for n, m in (("c1", "c1"), ("c2", "c2"), ("c3", "fwd"), ("c4", "varlen"),
                                                   ("c5", "decode")) if m in ms}
        res["cpu_baseline"] = cpu_baseline({"c1": w1, "c2": w2, "c3": w3, "c4": w4, "c5": w5}, gpu,
                                           {"c1": 1.0, "c2": 3.0, "c3": 10.0, "c4": 6.0, "c5": 4.0})
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
