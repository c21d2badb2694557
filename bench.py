"""Benchmark of the RoPE + causal GQA attention path on one MI355X.

One step = one pass of the hot path over the workload's synthetic batch:
  * prefill (headline): the GQA workload at full size -- B=1, Hq=64, Hkv=8, S=8192, D=128,
    bf16 inputs, causal, RoPE base 10000 fused into the Q/K tile loads; one attn_prefill launch;
  * decode: batch 32 against an 8192-token cache, Hq=64, Hkv=8, D=128, query rotated at 8192;
    one attn_decode call (split + merge launches);
  * long (optional, --long): the 32k-token prefill with 1% of keys scaled by 8.

Inputs are resident in HBM before timing starts.  Warmup launches, then K timed launches
bracketed by torch.cuda.synchronize(), timed with HIP events recorded on the stream the
library launches on (torch's current stream).  Prints ONE JSON line on stdout.

``value`` is prefill TFLOP/s with FLOPs = 2*B*Hq*S^2*D (the causal half of QK^T and PV).
The decode figure is K/V bytes read (2*B*Hkv*L*D*2 = 1 GiB) per second.  ``cpu_baseline``
times the fp64 oracle on a bounded sample of query rows of the same workload on the host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16/fp16 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E peak

# HBM bytes measured by rocprofv3 --pmc (FETCH_SIZE / WRITE_SIZE per dispatch, scaled by the
# copy-kernel calibration factor); None until counters are taken for the current kernels.
MEASURED_TRAFFIC = {"prefill_gqa": None, "decode": None}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--long", action="store_true", help="also time the 32k long-context prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "long", "all"], default="all")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def time_launches(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps   # ms per call


def bench_prefill(lib, inputs, wl, steps, warmup, variants=True):
    """Times one prefill step (keys rotated once into a workspace + the attention kernel), and
    separately the attention kernel alone, the key-rotation pass alone and the fused variant."""
    import torch
    log(f"[bench] generating {wl.name} prefill inputs B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} S={wl.S} D={wl.D}")
    p = inputs.make_prefill(wl)
    q, k, v = p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda")
    tab = lib.make_rope_table(wl.S, wl.D)
    out = torch.empty_like(q)
    ws = torch.empty(lib.prefill_workspace_bytes(wl.B, wl.Hkv, wl.S, wl.D), dtype=torch.uint8, device="cuda")
    krot = ws.view(torch.float16).view(k.shape)
    torch.cuda.synchronize()
    flops = wl.prefill_flops()
    log(f"[bench] timing {wl.name} prefill step: warmup {warmup}, steps {steps}")
    r = {"p": p}
    r["ms_step"] = time_launches(lambda: lib.prefill(q, k, v, tab, out=out, workspace=ws), steps, warmup)
    if variants:
        r["ms_kernel"] = time_launches(lambda: lib.prefill_prerotated(q, krot, v, tab, out=out), steps, warmup)
        r["ms_rope"] = time_launches(lambda: lib.rotate_keys_f16(k, tab, out=krot), steps, warmup)
        r["ms_fused"] = time_launches(lambda: lib.prefill(q, k, v, tab, out=out), steps, warmup)
    for key in ("ms_step", "ms_kernel", "ms_fused"):
        if key in r:
            r[key.replace("ms_", "tflops_")] = flops / (r[key] * 1e-3) / 1e12
    log(f"[bench] {wl.name} prefill: " + ", ".join(f"{k_}={v_:.4f}" for k_, v_ in r.items() if k_ != "p"))
    return r


def bench_decode(lib, inputs, wl, steps, warmup):
    import torch
    log(f"[bench] generating decode inputs B={wl.B} cache={wl.S} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D}")
    d = inputs.make_decode(wl)
    q, kc, vc = d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda")
    cl = torch.from_numpy(d.cache_len).cuda()
    qp = torch.from_numpy(d.q_pos).cuda()
    tab = lib.make_rope_table(int(d.q_pos.max()) + 1, wl.D)
    out = torch.empty_like(q)
    ws = torch.empty(lib.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.S, wl.D, 0), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] timing decode: warmup {warmup}, steps {steps}")
    ms = time_launches(lambda: lib.decode(q, kc, vc, cl, qp, tab, out=out, workspace=ws), steps, warmup)
    nbytes = wl.decode_kv_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode: {ms:.4f} ms/call, {gbs:.1f} GB/s of K/V")
    return d, ms, gbs


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        n = 1
    return int(n)


def cpu_baseline_prefill(p, target_s=12.0):
    """Time the fp64 oracle on seeded query rows of the same workload (all heads)."""
    import oracle
    wl = p.wl
    rng = np.random.default_rng(1234)

    def run(nrows):
        rows = np.stack([np.sort(rng.choice(wl.S, size=nrows, replace=False)) for _ in range(wl.Hq)])
        t0 = time.perf_counter()
        oracle.attention(p.q.f32, p.k.f32, p.v.f32, causal=True, rope_base=wl.rope_base, rows=rows)
        dt = time.perf_counter() - t0
        flops = float(np.sum(4.0 * wl.D * (rows + 1))) * wl.B   # causal work of the sampled rows
        return dt, flops, rows.shape[1]

    dt, flops, n = run(16)
    if dt < target_s / 4:
        n2 = int(min(wl.S, max(16, 16 * target_s / max(dt, 1e-3))))
        dt, flops, n = run(n2)
    tflops = flops / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{n} seeded query rows per head x {wl.Hq} heads of the {wl.name} workload "
                      f"(S={wl.S}), fp64 NumPy, {dt:.2f} s wall; FLOPs counted as 4*D*(i+1) per row",
            "wall_s": dt, "host_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline_decode(d, target_s=6.0):
    import oracle
    wl = d.wl
    t0 = time.perf_counter()
    nb = 1
    oracle.decode(d.q.f32[:nb], d.k_cache.f32[:nb], d.v_cache.f32[:nb], d.cache_len[:nb], d.q_pos[:nb])
    dt = time.perf_counter() - t0
    if dt < target_s / 4:
        nb = int(min(wl.B, max(1, target_s / max(dt, 1e-3))))
        t0 = time.perf_counter()
        oracle.decode(d.q.f32[:nb], d.k_cache.f32[:nb], d.v_cache.f32[:nb], d.cache_len[:nb], d.q_pos[:nb])
        dt = time.perf_counter() - t0
    nbytes = 2 * nb * wl.Hkv * wl.S * wl.D * 2
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{nb} of {wl.B} sequences (all heads, full cache), fp64 NumPy, {dt:.2f} s wall; "
                      f"bytes = bf16 K/V of those sequences"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in the design document); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from transformer_self_attention_amd import inputs, lib

    W = inputs.WORKLOADS
    res = {}
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only in ("prefill", "all"):
        res["prefill"] = bench_prefill(lib, inputs, W["gqa"], args.steps, args.warmup)
    if args.only in ("decode", "all"):
        res["decode"] = bench_decode(lib, inputs, W["decode"], args.steps, args.warmup)
    if args.long or args.only == "long":
        res["long"] = bench_prefill(lib, inputs, W["long"], max(2, args.steps // 4), min(args.warmup, 2),
                                    variants=False)

    out = {
        "metric": "causal GQA prefill TFLOP/s (% MFMA peak); decode KV-read GB/s (% HBM peak)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
    }
    if "prefill" in res:
        r = res["prefill"]
        p, ms, tflops = r["p"], r["ms_step"], r["tflops_step"]
        kern_tflops = r.get("tflops_kernel", tflops)
        wl = p.wl
        out.update({
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "step_parts": {"rotate_keys_f16_ms": round(r.get("ms_rope", float("nan")), 5),
                           "attention_kernel_ms": round(r.get("ms_kernel", float("nan")), 5),
                           "fused_rope_variant_ms": round(r.get("ms_fused", float("nan")), 5),
                           "fused_rope_variant_tflops": round(r.get("tflops_fused", float("nan")), 2)},
            "operand_dtypes": {"inputs": "bf16", "qk_mfma": "f16", "pv_mfma": "bf16", "accumulate": "f32",
                               "output": "bf16"},
            "config": {"workload": "GQA causal prefill with fused RoPE", "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv,
                       "seq_len": wl.S, "head_dim": wl.D, "causal": True, "rope_base": wl.rope_base,
                       "flops_per_step": wl.prefill_flops()},
            "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel (pre-rotated keys)",
                         "achieved": round(kern_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": MEASURED_TRAFFIC["prefill_gqa"]},
        })
    if "decode" in res:
        d, ms, gbs = res["decode"]
        wl = d.wl
        dec = {"metric": "decode KV-read GB/s", "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 5),
               "config": {"workload": "batch decode against a KV cache", "B": wl.B, "cache_len": wl.S,
                          "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.D, "kv_bytes_per_step": wl.decode_kv_bytes()},
               "roofline": {"bound": "hbm", "kernel": "decode_split_kernel + decode_merge_kernel",
                            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": MEASURED_TRAFFIC["decode"]}}
        if "prefill" not in res:
            out.update({"value": dec["value"], "unit": "GB/s", "ms_per_step": dec["ms_per_step"],
                        "config": dec["config"], "roofline": dec["roofline"]})
        out["decode"] = dec
    if "long" in res:
        r = res["long"]
        p, ms, tflops = r["p"], r["ms_step"], r["tflops_step"]
        out["long_prefill"] = {"value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
                               "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                               "config": {"B": p.wl.B, "Hq": p.wl.Hq, "Hkv": p.wl.Hkv, "seq_len": p.wl.S,
                                          "head_dim": p.wl.D, "big_key_frac": p.wl.big_key_frac}}
    if not args.no_cpu_baseline:
        if "prefill" in res:
            log("[bench] timing the fp64 oracle on the host (cpu_baseline, prefill sample)")
            out["cpu_baseline"] = cpu_baseline_prefill(res["prefill"]["p"])
        if "decode" in res:
            log("[bench] timing the fp64 oracle on the host (cpu_baseline, decode sample)")
            cb = cpu_baseline_decode(res["decode"][0])
            if "prefill" in res:
                out["decode"]["cpu_baseline"] = cb
            else:
                out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
