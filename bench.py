#!/usr/bin/env python3
"""Throughput of the TurboQuant codec on one MI355X.

One step = the codec hot path over the bulk-prefill workload: encode K (4-bit)
and V (2-bit) of 32 layers x 8 KV heads x 32768 tokens x head_dim 128 (bf16
AR(1)-correlated rows with outlier channels) in one launch, then decode both
back to fp32 (two launches).  `value` is the whole step's algorithmic bytes
per second (inputs already resident in HBM).  The same run also times the
fused decode-step attention (batch 32, 32 query / 8 KV heads, head_dim 128,
context 16384, K4/V2) and reports its microseconds per step, and times the
oracle on a bounded sample of the same codec workload on the host CPU.

Prints one JSON line.  Only --gpus 1 is supported (this build targets a
single GPU).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "codec GB/s & rows/s (K4/V2, d=128) as % HBM peak; tq_attn_decode µs/step"
HBM_PEAK_GBS = 8000.0
SEED = 42

# bulk prefill workload
L3, H3, T3, D3, BK3, BV3 = 32, 8, 32768, 128, 4, 2
# fused decode attention workload
B4, HQ4, HKV4, D4, T4, BK4, BV4 = 32, 32, 8, 128, 16384, 4, 2


def enc_bytes(n, d, bits, in_bytes):
    """algorithmic bytes of encoding n rows: input + packed + fp32 norm"""
    return n * (d * in_bytes + d * bits // 8 + 4)


def dec_bytes(n, d, bits):
    """algorithmic bytes of decoding n rows: packed + norm + fp32 output"""
    return n * (d * bits // 8 + 4 + 4 * d)


def attn_bytes(B, Hq, Hkv, d, T, bk, bv):
    """packed K and V rows with their norms, plus q (bf16) in and out (fp32)"""
    return B * Hkv * T * (d * bk // 8 + 4 + d * bv // 8 + 4) + B * Hq * d * (2 + 4)


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_vector_rotate_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain 1 GiB device copy, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))


def cpu_baseline(sample_rows: int, threads: int):
    """Oracle (plain fp64 C) encode + decode of a sample of the bulk-prefill
    rows, rows split statically over `threads` host threads."""
    import numpy as np
    import kvgen
    import oracle
    tokens = max(sample_rows // (H3 * 2), 1)
    k = kvgen.ar1_outliers((2, H3, tokens, D3), 3).float().numpy().reshape(-1, D3)
    v = kvgen.ar1_outliers((2, H3, tokens, D3), 103).float().numpy().reshape(-1, D3)
    oracle.codebook_float(D3, BK3)
    oracle.codebook_float(D3, BV3)

    def job(args):
        x, bits = args
        p, n = oracle.encode(x, D3, bits, SEED)
        oracle.decode(p, n, D3, bits, SEED)

    parts = [(c, BK3) for c in np.array_split(k, threads)] + \
            [(c, BV3) for c in np.array_split(v, threads)]
    t0, c0 = time.perf_counter(), time.process_time()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, parts))
    dt, cpu_s = time.perf_counter() - t0, time.process_time() - c0
    n = k.shape[0]
    nbytes = (enc_bytes(n, D3, BK3, 2) + enc_bytes(n, D3, BV3, 2)
              + dec_bytes(n, D3, BK3) + dec_bytes(n, D3, BV3))
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} K rows + {n} V rows of the bulk-prefill workload (2 layers x 8 heads x "
                      f"{tokens} tokens), encode + decode, {dt:.2f} s wall, {cpu_s:.1f} s of CPU time",
            "rows_per_s": 2 * n / dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--attn-reps", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1 << 22)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    import kvgen
    import kv_cache_vector_rotate_amd as tq

    # ---------------- codec step: encode K4/V2 + decode both
    n = L3 * H3 * T3
    print(f"bench: generating {n} K and V rows (bf16)", file=sys.stderr, flush=True)
    k = kvgen.ar1_outliers((L3, H3, T3, D3), 3, "cuda")
    v = kvgen.ar1_outliers((L3, H3, T3, D3), 103, "cuda")
    kp = torch.empty(n, D3 * BK3 // 8, dtype=torch.uint8, device="cuda")
    vp = torch.empty(n, D3 * BV3 // 8, dtype=torch.uint8, device="cuda")
    kn = torch.empty(n, dtype=torch.float32, device="cuda")
    vn = torch.empty(n, dtype=torch.float32, device="cuda")
    ko = torch.empty(n, D3, dtype=torch.float32, device="cuda")
    vo = torch.empty(n, D3, dtype=torch.float32, device="cuda")
    names = ["encode_k4v2", "decode_k4", "decode_v2"]
    nbytes = {"encode_k4v2": enc_bytes(n, D3, BK3, 2) + enc_bytes(n, D3, BV3, 2),
              "decode_k4": dec_bytes(n, D3, BK3), "decode_v2": dec_bytes(n, D3, BV3)}
    step_bytes = sum(nbytes.values())

    def settle(fn=None, seconds=0.3):
        # untimed: a freshly started GPU runs its first ~0.1 s of work at a
        # lower clock; repeat the work until the clock has settled
        t = time.perf_counter()
        while time.perf_counter() - t < seconds:
            (fn or step)()
            torch.cuda.synchronize()

    def step(ev=None):
        if ev: ev[0].record()
        tq.tq_encode(k, v, BK3, BV3, SEED, kp, kn, vp, vn)
        if ev: ev[1].record()
        tq.tq_decode(kp, kn, D3, BK3, SEED, out=ko)
        if ev: ev[2].record()
        tq.tq_decode(vp, vn, D3, BV3, SEED, out=vo)
        if ev: ev[3].record()

    settle()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {nm: [] for nm in names}
    for ev in evs:
        for j, nm in enumerate(names):
            per[nm].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
    kern = {}
    for nm in names:
        avg = sum(per[nm]) / len(per[nm])
        kern[nm] = {"avg_us": avg * 1e6, "min_us": min(per[nm]) * 1e6,
                    "alg_bytes": nbytes[nm], "GB_s": nbytes[nm] / avg / 1e9,
                    "pct_hbm_peak": 100 * nbytes[nm] / avg / 1e9 / HBM_PEAK_GBS}
    del ko, vo
    value = step_bytes * args.steps / wall / 1e9
    dom = max(names, key=lambda nm: kern[nm]["avg_us"])

    # ---------------- fused decode attention, two caches alternated (> MALL)
    print("bench: attention cache", file=sys.stderr, flush=True)
    caches = []
    for c in range(2):
        cache = tq.TQCache(1, B4, HKV4, T4, D4, BK4, BV4, SEED)
        kk = kvgen.normal((B4, HKV4, T4, D4), 4 + 10 * c, "cuda")
        vv = kvgen.normal((B4, HKV4, T4, D4), 5 + 10 * c, "cuda")
        tq.tq_encode(kk, vv, BK4, BV4, SEED, cache.k_packed[0], cache.k_norms[0],
                     cache.v_packed[0], cache.v_norms[0])
        del kk, vv
        caches.append(cache)
    q = kvgen.normal((B4, HQ4, D4), 44, "cuda", torch.bfloat16)
    out = torch.empty(B4, HQ4, D4, dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attn_workspace_bytes(caches[0], 0, HQ4, T4), dtype=torch.uint8,
                     device="cuda")
    settle(lambda: [tq.tq_attn_decode(caches[i % 2], 0, q, T4, out=out, workspace=ws)
                    for i in range(4)], 0.2)
    for i in range(3):
        tq.tq_attn_decode(caches[i % 2], 0, q, T4, out=out, workspace=ws)
    torch.cuda.synchronize()
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.attn_reps)]
    for i, (a, b) in enumerate(aev):
        a.record()
        tq.tq_attn_decode(caches[i % 2], 0, q, T4, out=out, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    at = sorted(a.elapsed_time(b) * 1e3 for a, b in aev)
    attn_us = sum(at) / len(at)
    ab = attn_bytes(B4, HQ4, HKV4, D4, T4, BK4, BV4)
    # the same launch with the sparse-V gate at 1e-3 (N(0,1) keys: few rows gated)
    ws_g = torch.empty(tq.tq_attn_workspace_bytes(caches[0], 0, HQ4, T4, 1e-3),
                       dtype=torch.uint8, device="cuda")
    for i in range(3):
        tq.tq_attn_decode(caches[i % 2], 0, q, T4, out=out, workspace=ws_g, sparse_v=1e-3)
    for i, (a, b) in enumerate(aev):
        a.record()
        tq.tq_attn_decode(caches[i % 2], 0, q, T4, out=out, workspace=ws_g, sparse_v=1e-3)
        b.record()
    torch.cuda.synchronize()
    ats = [a.elapsed_time(b) * 1e3 for a, b in aev]
    attn_sparse_us = sum(ats) / len(ats)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "bulk prefill codec step: encode K4/V2 (one launch) + decode K and V, "
                        "32 layers x 8 KV heads x 32768 tokens, head_dim 128, bf16 AR(1) rho 0.6 "
                        "rows with 4 outlier channels x8 per head, sign seed 42",
            "rows_per_step": 2 * n,
            "alg_bytes_per_step": step_bytes,
        },
        "rows_per_s": round(2 * n * args.steps / wall, 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels": {nm: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                         for kk, vv in kern[nm].items()} for nm in names},
        "attn_us_per_step": round(attn_us, 2),
        "attn": {
            "workload": "tq_attn_decode batch 32, 32 query heads on 8 KV heads, head_dim 128, "
                        "context 16384, K4/V2, bf16 q, two caches alternated",
            "median_us": round(at[len(at) // 2], 2), "min_us": round(at[0], 2),
            "alg_bytes": ab, "GB_s": round(ab / attn_us / 1e3, 1),
            "pct_hbm_peak": round(100 * ab / attn_us / 1e3 / HBM_PEAK_GBS, 2),
            "sparse_v_1e-3_us": round(attn_sparse_us, 2),
        },
        "roofline": {
            "bound": "hbm", "kernel": dom,
            "achieved": round(kern[dom]["GB_s"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern[dom]["GB_s"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(dom),
        },
    }
    if not args.no_cpu_baseline:
        print("bench: oracle CPU baseline", file=sys.stderr, flush=True)
        threads = min(16, os.cpu_count() or 1)
        res["cpu_baseline"] = cpu_baseline(args.cpu_sample_rows, threads)
        res["cpu_baseline"]["value"] = round(res["cpu_baseline"]["value"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
