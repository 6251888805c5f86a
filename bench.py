#!/usr/bin/env python3
"""Benchmark of the packed varlen attention hot path on one MI355X.

A step is one forward call over one batch of seeded synthetic input that is
already resident in HBM.  Default workload: packed full-causal GQA forward,
bf16, 8192 tokens in documents of 128..2048 tokens, 32 query / 8 KV heads,
head_dim 128.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--copy-calibration MiB]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sliding_window_gqa_varlen_amd import metrics, workloads as W  # noqa: E402

DENSE_SOURCES = ["sliding_window_gqa_varlen_amd/csrc/dense_fwd.hip", "sliding_window_gqa_varlen_amd/csrc/dense_common.h",
                 "sliding_window_gqa_varlen_amd/csrc/device_common.h"]
SPARSE_SOURCES = ["sliding_window_gqa_varlen_amd/csrc/sparse_mla_fwd.hip",
                  "sliding_window_gqa_varlen_amd/csrc/device_common.h"]
BWD_SOURCES = ["sliding_window_gqa_varlen_amd/csrc/dense_bwd.hip", "sliding_window_gqa_varlen_amd/csrc/dense_common.h",
               "sliding_window_gqa_varlen_amd/csrc/device_common.h"]
VPROJ_SOURCES = ["sliding_window_gqa_varlen_amd/csrc/mla_value_proj.hip",
                 "sliding_window_gqa_varlen_amd/csrc/device_common.h"]
TRAFFIC_FILES = {
    "causal_gqa_bf16_t8192": "profiles/dense_fwd_causal_gqa_bf16_t8192_traffic.txt",
    "swa1024_gqa_bf16_t32768": "profiles/dense_fwd_swa1024_gqa_bf16_t32768_traffic.txt",
    "swa128_sink_gqa_bf16_t65536": "profiles/dense_fwd_swa128_sink_gqa_bf16_t65536_traffic.txt",
    "causal_gqa_d256_bf16_t8192": "profiles/dense_fwd_causal_gqa_d256_bf16_t8192_traffic.txt",
    "causal_gqa_bwd_bf16_t8192": "profiles/dense_bwd_causal_gqa_bf16_t8192_traffic.txt",
    "swa1024_gqa_bwd_bf16_t32768": "profiles/dense_bwd_swa1024_gqa_bf16_t32768_traffic.txt",
    "swa128_sink_gqa_bwd_bf16_t65536": "profiles/dense_bwd_swa128_sink_gqa_bf16_t65536_traffic.txt",
    "sparse_mla_bf16_t16384": "profiles/sparse_mla_fwd_bf16_t16384_traffic.txt",
    "sparse_mla_nope_bf16_t16384": "profiles/sparse_mla_fwd_nope_bf16_t16384_traffic.txt",
    "mla_value_proj_bf16_t16384": "profiles/mla_value_proj_bf16_t16384_traffic.txt",
}


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(name: str, sources) -> float | None:
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the sources."""
    path = TRAFFIC_FILES.get(name)
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    with open(os.path.join(ROOT, path)) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != sources_sha256(sources):
        return None  # the kernel changed since the counters were taken
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline_dense(inp, min_s: float = 10.0, max_s: float = 30.0) -> dict:
    """The fp64 oracle as it stands, timed document by document.

    Whole passes over the documents repeat until at least ``min_s`` seconds are
    timed; a pass stops early once ``max_s`` is spent.
    """
    import oracle
    cu = inp["cu_seqlens"]
    w = inp["workload"]
    n_docs = len(cu) - 1
    done, t_total, passes = [], 0.0, 0
    while t_total < min_s:
        for d in range(n_docs):
            s, e = int(cu[d]), int(cu[d + 1])
            sl = slice(s, e)
            t = time.perf_counter()
            oracle.varlen_attn_ref(inp["q"][sl], inp["k"][sl], inp["v"][sl], [0, e - s], inp["window"],
                                   inp["scale"], inp["sinks"])
            t_total += time.perf_counter() - t
            done.append(e - s)
            if t_total >= max_s:
                break
        passes += 1
        if t_total >= max_s:
            break
    flops = metrics.dense_flops(done, inp["window"], w.Hq, w.D)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle, {len(done)} document calls ({passes} pass(es) over the {n_docs} "
                      f"documents of the workload, all {w.Hq} heads), {t_total:.1f} s on {cpu_model()}"}


def cpu_baseline_dense_bwd(inp, min_s: float = 10.0, max_s: float = 30.0) -> dict:
    """The fp64 backward oracle as it stands, document by document (as the forward's leg)."""
    import oracle
    cu = inp["cu_seqlens"]
    w = inp["workload"]
    do = W.make_dout(w.seed, inp["q"].shape)
    done, t_total, passes = [], 0.0, 0
    while t_total < min_s:
        for d in range(len(cu) - 1):
            s, e = int(cu[d]), int(cu[d + 1])
            sl = slice(s, e)
            t = time.perf_counter()
            oracle.varlen_attn_bwd_ref(inp["q"][sl], inp["k"][sl], inp["v"][sl], do[sl], [0, e - s], inp["window"],
                                       inp["scale"], inp["sinks"])
            t_total += time.perf_counter() - t
            done.append(e - s)
            if t_total >= max_s:
                break
        passes += 1
        if t_total >= max_s:
            break
    flops = metrics.dense_bwd_flops(done, inp["window"], w.Hq, w.D)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy backward oracle, {len(done)} document calls ({passes} pass(es) over the "
                      f"{len(cu) - 1} documents, all {w.Hq} heads), {t_total:.1f} s on {cpu_model()}"}


def cpu_baseline_sparse(inp, budget_s: float = 20.0) -> dict:
    import oracle
    w = inp["workload"]
    T = w.T
    rng = np.random.default_rng(0)
    order = rng.permutation(T)
    done, t_total = [], 0.0
    for start in range(0, T, 16):
        toks = order[start:start + 16]
        t = time.perf_counter()
        oracle.sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                   inp["scale"], toks)
        t_total += time.perf_counter() - t
        done.extend(toks.tolist())
        if t_total >= budget_s:
            break
    sub_idx = inp["indices"][np.array(done)]
    # valid slots of the sampled rows, then the same byte formula per sampled token
    valid = 0
    for r, t in enumerate(done):
        row = sub_idx[r].astype(np.int64)
        ok = (row >= 0) & (row < T) & (row <= t)
        ok &= inp["doc_ids"][np.where(ok, row, 0)] == inp["doc_ids"][t]
        valid += int(ok.sum())
    nbytes = metrics.sparse_bytes(valid, len(done), w.H, w.d_latent, w.d_rope, w.topk)
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle over {len(done)} random tokens of {T}, {t_total:.1f} s on {cpu_model()}"}


def cpu_baseline_vproj(inp, budget_s: float = 15.0) -> dict:
    import oracle
    w = inp["workload"]
    rng = np.random.default_rng(0)
    done, t_total, nbytes = 0, 0.0, 0
    while t_total < budget_s:
        t0 = int(rng.integers(0, w.T - 256 + 1))
        t = time.perf_counter()
        oracle.mla_value_proj_ref(inp["o_latent"][t0:t0 + 256], inp["value_weight"])
        t_total += time.perf_counter() - t
        done += 256
        nbytes += metrics.value_proj_bytes(256, w.H, w.d_latent, w.d_value)
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle over {done // 256} random runs of 256 tokens of {w.T} (all {w.H} heads), "
                      f"{t_total:.1f} s on {cpu_model()}"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="causal_gqa_bf16_t8192",
                    choices=[w.name for w in W.WORKLOADS + W.EXTRA_WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path runs per GPU with no collectives).", file=sys.stderr)
        return 2

    import torch
    from sliding_window_gqa_varlen_amd import binding

    binding.load_library()  # raises when the HIP library is missing: there is no fallback path
    dev = torch.device("cuda:0")
    wl = next(w for w in W.WORKLOADS + W.EXTRA_WORKLOADS if w.name == args.workload)
    sparse = isinstance(wl, W.SparseWorkload)
    vproj = isinstance(wl, W.ValueProjWorkload)

    if vproj:
        inp = W.make_value_proj(wl)
        o_lat = torch.from_numpy(inp["o_latent"]).to(dev).to(torch.bfloat16)
        vw = torch.from_numpy(inp["value_weight"]).to(dev).to(torch.bfloat16)
        out = torch.empty(wl.T, wl.H, wl.d_value, device=dev, dtype=torch.bfloat16)

        def step():
            binding.mla_value_proj(o_lat, vw, out=out)

        work = metrics.value_proj_bytes(wl.T, wl.H, wl.d_latent, wl.d_value)
        flops = metrics.value_proj_flops(wl.T, wl.H, wl.d_latent, wl.d_value)
        sources = VPROJ_SOURCES
        dtype = "bf16"
        config = {"workload": wl.name, "tokens": wl.T, "heads": wl.H, "d_latent": wl.d_latent,
                  "d_value": wl.d_value}
    elif getattr(wl, "backward", False):
        inp = W.make_dense(wl)
        q, k, v = (torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v"))
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
        sinks = None if inp["sinks"] is None else torch.from_numpy(inp["sinks"]).to(dev)
        o_fwd, lse = binding.varlen_attn_fwd(q, k, v, cu, inp["n_docs"], wl.window, wl.scale, sinks)
        dout = torch.from_numpy(W.make_dout(wl.seed, inp["q"].shape)).to(dev).to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(wl.T, wl.Hq, device=dev, dtype=torch.float32)
        dsinks = None if sinks is None else torch.empty(wl.Hq, device=dev, dtype=torch.float32)

        def step():
            binding.varlen_attn_bwd(q, k, v, o_fwd, dout, lse, cu, inp["n_docs"], wl.window, wl.scale, sinks,
                                    dq=dq, dk=dk, dv=dv, dsinks=dsinks, delta=delta)

        flops = metrics.dense_bwd_flops(inp["lengths"], wl.window, wl.Hq, wl.D)
        work = flops
        sources = BWD_SOURCES
        dtype = "bf16"
        config = {"workload": wl.name, "tokens": wl.T, "documents": inp["n_docs"], "q_heads": wl.Hq,
                  "kv_heads": wl.Hkv, "head_dim": wl.D, "window": wl.window, "sinks": wl.sinks,
                  "allowed_pairs": metrics.dense_allowed_pairs(inp["lengths"], wl.window),
                  "kernels": "delta, dq, dk/dv (one varlen_attn_bwd call)"}
    elif sparse:
        inp = W.make_sparse(wl)
        q = torch.from_numpy(inp["q"]).to(dev).to(torch.bfloat16)
        lat = torch.from_numpy(inp["latent"]).to(dev).to(torch.bfloat16)
        kpe = torch.from_numpy(inp["k_pe"]).to(dev).to(torch.bfloat16)
        idx = torch.from_numpy(inp["indices"]).to(dev)
        ids = torch.from_numpy(inp["doc_ids"]).to(dev)
        out = torch.empty(wl.T, wl.H, wl.d_latent, device=dev, dtype=torch.bfloat16)
        lse = torch.empty(wl.T, wl.H, device=dev, dtype=torch.float32)

        def step():
            binding.sparse_mla_fwd(q, lat, kpe, idx, ids, wl.scale, out=out, lse=lse)

        valid = metrics.sparse_valid_slots(inp["indices"], inp["doc_ids"])
        work = metrics.sparse_bytes(valid, wl.T, wl.H, wl.d_latent, wl.d_rope, wl.topk)
        flops = metrics.sparse_flops(valid, wl.H, wl.d_latent, wl.d_rope)
        sources = SPARSE_SOURCES
        dtype = "bf16"
        config = {"workload": wl.name, "tokens": wl.T, "heads": wl.H, "d_latent": wl.d_latent,
                  "d_rope": wl.d_rope, "topk": wl.topk, "valid_slots": valid, "documents": len(inp["lengths"])}
    else:
        inp = W.make_dense(wl)
        td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        q = torch.from_numpy(inp["q"]).to(dev).to(td)
        k = torch.from_numpy(inp["k"]).to(dev).to(td)
        v = torch.from_numpy(inp["v"]).to(dev).to(td)
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
        sinks = None if inp["sinks"] is None else torch.from_numpy(inp["sinks"]).to(dev)
        out = torch.empty(wl.T, wl.Hq, wl.D, device=dev, dtype=td)
        lse = torch.empty(wl.T, wl.Hq, device=dev, dtype=torch.float32)

        def step():
            binding.varlen_attn_fwd(q, k, v, cu, inp["n_docs"], wl.window, wl.scale, sinks, out=out, lse=lse)

        flops = metrics.dense_flops(inp["lengths"], wl.window, wl.Hq, wl.D)
        work = flops
        sources = DENSE_SOURCES
        dtype = wl.dtype
        config = {"workload": wl.name, "tokens": wl.T, "documents": inp["n_docs"], "q_heads": wl.Hq,
                  "kv_heads": wl.Hkv, "head_dim": wl.D, "window": wl.window, "sinks": wl.sinks,
                  "allowed_pairs": metrics.dense_allowed_pairs(inp["lengths"], wl.window)}

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()  # the library launches on this stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / max(args.steps, 1)

    # per-launch spread: a separate pass of individually timed launches (not part of `value`)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    launch_us = {"median": per[len(per) // 2], "min": per[0], "max": per[-1], "launches": len(per)}

    # sparse: the 18.9 MB key table otherwise stays in the Infinity Cache between launches; a
    # cold launch follows a 512 MiB write that evicts it (separate pass, not part of `value`)
    cold_us = None
    if sparse:
        flush = torch.empty(512 << 20, device=dev, dtype=torch.uint8)
        cold = []
        for _ in range(5):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        del flush
        cold_us = sorted(cold)[len(cold) // 2]

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    traffic = committed_traffic(wl.name, sources)
    if vproj:
        achieved = work / (ms * 1e-3) / 1e9
        value = achieved
        roof = metrics.roofline("hbm", achieved, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
        metric, unit = "sparse MLA value up-projection algorithmic HBM GB/s (1 GPU)", "GB/s"
    elif getattr(wl, "backward", False):
        achieved = flops / (ms * 1e-3) / 1e12
        value = achieved
        min_bytes = metrics.dense_bwd_min_bytes(wl.T, wl.Hq, wl.Hkv, wl.D, inp["n_docs"], wl.sinks)
        hbm_gbps = min_bytes / (ms * 1e-3) / 1e9
        # the roofline that binds, as for the forward
        if flops / min_bytes < metrics.MI355X_BF16_DENSE_TFLOPS * 1e12 / (metrics.MI355X_HBM_GBPS * 1e9):
            roof = metrics.roofline("hbm", hbm_gbps, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
        else:
            roof = metrics.roofline("mfma", achieved, metrics.MI355X_BF16_DENSE_TFLOPS, "TFLOP/s", traffic)
        metric, unit = "packed GQA attn bwd mask-effective TFLOP/s + % bf16 MFMA peak (1 GPU)", "TFLOP/s"
        config["pct_bf16_mfma_peak"] = 100.0 * achieved / metrics.MI355X_BF16_DENSE_TFLOPS
        config["min_hbm_gbps"] = hbm_gbps
        config["arithmetic_intensity"] = flops / min_bytes
    elif sparse:
        achieved = work / (ms * 1e-3) / 1e9
        value = achieved
        roof = metrics.roofline("hbm", achieved, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
        metric, unit = "sparse MLA fwd algorithmic HBM GB/s (1 GPU)", "GB/s"
    else:
        achieved = flops / (ms * 1e-3) / 1e12
        value = achieved
        peak = metrics.MI355X_BF16_DENSE_TFLOPS if wl.dtype == "bf16" else metrics.MI355X_FP32_MFMA_TFLOPS
        min_bytes = metrics.dense_min_bytes(wl.T, wl.Hq, wl.Hkv, wl.D, 2 if wl.dtype == "bf16" else 4,
                                            inp["n_docs"], True, wl.sinks)
        hbm_gbps = min_bytes / (ms * 1e-3) / 1e9
        # the roofline that binds: HBM when the arithmetic intensity is below the ridge point
        if flops / min_bytes < peak * 1e12 / (metrics.MI355X_HBM_GBPS * 1e9):
            roof = metrics.roofline("hbm", hbm_gbps, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
        else:
            roof = metrics.roofline("mfma", achieved, peak, "TFLOP/s", traffic)
        metric, unit = "packed GQA attn fwd mask-effective TFLOP/s + % bf16 MFMA peak (1 GPU)", "TFLOP/s"
        config["pct_bf16_mfma_peak"] = 100.0 * achieved / metrics.MI355X_BF16_DENSE_TFLOPS
        config["min_hbm_gbps"] = hbm_gbps
        config["arithmetic_intensity"] = flops / min_bytes
    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded generator, inputs resident in HBM)",
        "config": config, "roofline": roof,
        "cpu_baseline": None,
    }
    if sparse or vproj:
        line["config"]["tflops"] = flops / (ms * 1e-3) / 1e12
    line["launch_us"] = launch_us
    if cold_us is not None:
        line["cold"] = {"us": cold_us, "value": work / (cold_us * 1e-6) / 1e9, "unit": unit,
                        "note": "median of 5 launches, each after a 512 MiB device write that evicts the key table"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline_vproj(inp) if vproj else
                                cpu_baseline_sparse(inp) if sparse else
                                cpu_baseline_dense_bwd(inp) if getattr(wl, "backward", False) else
                                cpu_baseline_dense(inp))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
