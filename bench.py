#!/usr/bin/env python3
"""Benchmark of the packed varlen attention hot path on one MI355X.

A step is one forward call over one batch of seeded synthetic input that is already resident
in HBM.  The headline workload (the line's `value`) is the packed full-causal GQA forward,
bf16, 8192 tokens in documents of 128..2048 tokens, 32 query / 8 KV heads, head_dim 128.

Default run: measured peaks (a bf16 MFMA-only loop, a streaming copy and read), then the
sliding-window (1024), learned-sink window-128 and sparse MLA workloads, then the headline,
each with 50 ms of untimed clock-ramp steps, W untimed warm-up steps and exactly K timed
steps, back to back on the GPU; then the fp64 oracle on the host for each (time-capped).
One JSON line: the headline's fields at the top level, the other workloads under "configs",
the probes under "measured_peaks".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--copy-calibration MiB]

--workload NAME times that one workload alone (profiling runs).
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


SUITE = ("swa1024_gqa_bf16_t32768", "swa128_sink_gqa_bf16_t65536", "sparse_mla_bf16_t16384")
# Untimed load before each case's warm-up steps: after idle the GPU's clocks take several
# milliseconds of load to rise (window 1024 measured 598 us per step after 5 warm-up steps of
# 2.5 ms, 512 us in steady state), so W steps alone may time the ramp.
CLOCK_RAMP_MS = 50.0
HEADLINE = "causal_gqa_bf16_t8192"


class Case:
    """One workload prepared on the GPU: its step, its algorithmic work and how to price it."""

    def __init__(self, wl, dev):
        import torch
        from sliding_window_gqa_varlen_amd import binding
        self.wl = wl
        self.kind = ("vproj" if isinstance(wl, W.ValueProjWorkload) else
                     "sparse" if isinstance(wl, W.SparseWorkload) else
                     "bwd" if getattr(wl, "backward", False) else "dense")
        if self.kind == "vproj":
            inp = W.make_value_proj(wl)
            o_lat = torch.from_numpy(inp["o_latent"]).to(dev).to(torch.bfloat16)
            vw = torch.from_numpy(inp["value_weight"]).to(dev).to(torch.bfloat16)
            out = torch.empty(wl.T, wl.H, wl.d_value, device=dev, dtype=torch.bfloat16)
            self.step = lambda: binding.mla_value_proj(o_lat, vw, out=out)
            self.work = metrics.value_proj_bytes(wl.T, wl.H, wl.d_latent, wl.d_value)
            self.flops = metrics.value_proj_flops(wl.T, wl.H, wl.d_latent, wl.d_value)
            self.sources, self.dtype = VPROJ_SOURCES, "bf16"
            self.config = {"workload": wl.name, "tokens": wl.T, "heads": wl.H, "d_latent": wl.d_latent,
                           "d_value": wl.d_value}
        elif self.kind == "bwd":
            inp = W.make_dense(wl)
            q, k, v = (torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v"))
            cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
            sinks = None if inp["sinks"] is None else torch.from_numpy(inp["sinks"]).to(dev)
            o_fwd, lse = binding.varlen_attn_fwd(q, k, v, cu, inp["n_docs"], wl.window, wl.scale, sinks)
            dout = torch.from_numpy(W.make_dout(wl.seed, inp["q"].shape)).to(dev).to(torch.bfloat16)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            delta = torch.empty(wl.T, wl.Hq, device=dev, dtype=torch.float32)
            dsinks = None if sinks is None else torch.empty(wl.Hq, device=dev, dtype=torch.float32)
            self.step = lambda: binding.varlen_attn_bwd(q, k, v, o_fwd, dout, lse, cu, inp["n_docs"], wl.window,
                                                        wl.scale, sinks, dq=dq, dk=dk, dv=dv, dsinks=dsinks,
                                                        delta=delta)
            self.flops = self.work = metrics.dense_bwd_flops(inp["lengths"], wl.window, wl.Hq, wl.D)
            self.min_bytes = metrics.dense_bwd_min_bytes(wl.T, wl.Hq, wl.Hkv, wl.D, inp["n_docs"], wl.sinks)
            self.sources, self.dtype = BWD_SOURCES, "bf16"
            self.config = {"workload": wl.name, "tokens": wl.T, "documents": inp["n_docs"], "q_heads": wl.Hq,
                           "kv_heads": wl.Hkv, "head_dim": wl.D, "window": wl.window, "sinks": wl.sinks,
                           "allowed_pairs": metrics.dense_allowed_pairs(inp["lengths"], wl.window),
                           "kernels": "delta, dq, dk/dv (one varlen_attn_bwd call)"}
        elif self.kind == "sparse":
            inp = W.make_sparse(wl)
            q = torch.from_numpy(inp["q"]).to(dev).to(torch.bfloat16)
            lat = torch.from_numpy(inp["latent"]).to(dev).to(torch.bfloat16)
            kpe = torch.from_numpy(inp["k_pe"]).to(dev).to(torch.bfloat16)
            idx = torch.from_numpy(inp["indices"]).to(dev)
            ids = torch.from_numpy(inp["doc_ids"]).to(dev)
            out = torch.empty(wl.T, wl.H, wl.d_latent, device=dev, dtype=torch.bfloat16)
            lse = torch.empty(wl.T, wl.H, device=dev, dtype=torch.float32)
            self.step = lambda: binding.sparse_mla_fwd(q, lat, kpe, idx, ids, wl.scale, out=out, lse=lse)
            valid = metrics.sparse_valid_slots(inp["indices"], inp["doc_ids"])
            self.work = metrics.sparse_bytes(valid, wl.T, wl.H, wl.d_latent, wl.d_rope, wl.topk)
            self.flops = metrics.sparse_flops(valid, wl.H, wl.d_latent, wl.d_rope)
            self.sources, self.dtype = SPARSE_SOURCES, "bf16"
            self.config = {"workload": wl.name, "tokens": wl.T, "heads": wl.H, "d_latent": wl.d_latent,
                           "d_rope": wl.d_rope, "topk": wl.topk, "valid_slots": valid,
                           "documents": len(inp["lengths"])}
        else:
            inp = W.make_dense(wl)
            td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
            q, k, v = (torch.from_numpy(inp[n]).to(dev).to(td) for n in ("q", "k", "v"))
            cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
            sinks = None if inp["sinks"] is None else torch.from_numpy(inp["sinks"]).to(dev)
            out = torch.empty(wl.T, wl.Hq, wl.D, device=dev, dtype=td)
            lse = torch.empty(wl.T, wl.Hq, device=dev, dtype=torch.float32)
            self.step = lambda: binding.varlen_attn_fwd(q, k, v, cu, inp["n_docs"], wl.window, wl.scale, sinks,
                                                        out=out, lse=lse)
            self.flops = self.work = metrics.dense_flops(inp["lengths"], wl.window, wl.Hq, wl.D)
            self.min_bytes = metrics.dense_min_bytes(wl.T, wl.Hq, wl.Hkv, wl.D, 2 if wl.dtype == "bf16" else 4,
                                                     inp["n_docs"], True, wl.sinks)
            self.sources, self.dtype = DENSE_SOURCES, wl.dtype
            self.config = {"workload": wl.name, "tokens": wl.T, "documents": inp["n_docs"], "q_heads": wl.Hq,
                           "kv_heads": wl.Hkv, "head_dim": wl.D, "window": wl.window, "sinks": wl.sinks,
                           "allowed_pairs": metrics.dense_allowed_pairs(inp["lengths"], wl.window)}
        inp["workload"] = wl
        self.inp = inp
        self.ms = None

    def timed(self, warmup: int, steps: int) -> float:
        """Untimed steps for CLOCK_RAMP_MS of wall time (the GPU's clocks rise over several
        milliseconds of load after idle), then W untimed steps, then exactly K steps between
        HIP events on the launch stream; ms per step."""
        import torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < CLOCK_RAMP_MS:
            for _ in range(4):
                self.step()
            torch.cuda.synchronize()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()  # the library launches on this stream
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            self.step()
        ev1.record(stream)
        torch.cuda.synchronize()
        self.ms = ev0.elapsed_time(ev1) / max(steps, 1)
        return self.ms

    def launch_spread(self, n: int = 20) -> dict:
        """Individually timed launches (a separate pass, not part of `value`)."""
        import torch
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            self.step()
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"median": per[len(per) // 2], "min": per[0], "max": per[-1], "launches": len(per)}

    def cold_us(self, dev) -> float:
        """Sparse: median of 5 launches, each after a 512 MiB device write that evicts the key table."""
        import torch
        stream = torch.cuda.current_stream()
        flush = torch.empty(512 << 20, device=dev, dtype=torch.uint8)
        cold = []
        for _ in range(5):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            self.step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        del flush
        return sorted(cold)[len(cold) // 2]

    def result(self, peaks: dict | None) -> dict:
        """metric, value, unit, roofline (against the published peak, with the measured one beside it)."""
        wl, ms = self.wl, self.ms
        traffic = committed_traffic(wl.name, self.sources)
        cfg = dict(self.config)
        mfma_meas = (peaks or {}).get("bf16_mfma_tflops")
        hbm_meas = (peaks or {}).get("copy_gbps")
        if self.kind in ("vproj", "sparse"):
            achieved = self.work / (ms * 1e-3) / 1e9
            roof = metrics.roofline("hbm", achieved, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
            roof["measured_peak"] = hbm_meas
            cfg["tflops"] = self.flops / (ms * 1e-3) / 1e12
            metric = ("sparse MLA value up-projection algorithmic HBM GB/s (1 GPU)" if self.kind == "vproj" else
                      "sparse MLA fwd algorithmic HBM GB/s (1 GPU)")
            unit = "GB/s"
        else:
            achieved = self.flops / (ms * 1e-3) / 1e12
            bf16 = self.dtype == "bf16"
            peak = metrics.MI355X_BF16_DENSE_TFLOPS if bf16 else metrics.MI355X_FP32_MFMA_TFLOPS
            hbm_gbps = self.min_bytes / (ms * 1e-3) / 1e9
            # the roofline that binds: HBM when the arithmetic intensity is below the ridge point
            if self.flops / self.min_bytes < peak * 1e12 / (metrics.MI355X_HBM_GBPS * 1e9):
                roof = metrics.roofline("hbm", hbm_gbps, metrics.MI355X_HBM_GBPS, "GB/s", traffic)
                roof["measured_peak"] = hbm_meas
            else:
                roof = metrics.roofline("mfma", achieved, peak, "TFLOP/s", traffic)
                roof["measured_peak"] = mfma_meas if bf16 else None
            cfg["pct_bf16_mfma_peak"] = 100.0 * achieved / metrics.MI355X_BF16_DENSE_TFLOPS
            cfg["min_hbm_gbps"] = hbm_gbps
            cfg["arithmetic_intensity"] = self.flops / self.min_bytes
            metric = ("packed GQA attn bwd mask-effective TFLOP/s + % bf16 MFMA peak (1 GPU)" if self.kind == "bwd"
                      else "packed GQA attn fwd mask-effective TFLOP/s + % bf16 MFMA peak (1 GPU)")
            unit = "TFLOP/s"
        if roof.get("measured_peak"):
            roof["frac_of_measured_peak"] = roof["achieved"] / roof["measured_peak"]
        return {"metric": metric, "value": achieved, "unit": unit, "ms_per_step": ms, "dtype": self.dtype,
                "config": cfg, "roofline": roof}

    def cpu_baseline(self, budget_s: float) -> dict:
        if self.kind == "vproj":
            return cpu_baseline_vproj(self.inp, budget_s=budget_s)
        if self.kind == "sparse":
            return cpu_baseline_sparse(self.inp, budget_s=budget_s)
        if self.kind == "bwd":
            return cpu_baseline_dense_bwd(self.inp, min_s=budget_s, max_s=3 * budget_s)
        return cpu_baseline_dense(self.inp, min_s=budget_s, max_s=3 * budget_s)


def measure_peaks(dev) -> dict:
    """Achievable peaks of this device from the library's probes (median of 5 launches each)."""
    import torch
    from sliding_window_gqa_varlen_amd import binding
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, device=dev, dtype=torch.float32)

    def time_it(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            amount = fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(amount / (a.elapsed_time(b) * 1e-3))
        return sorted(out)[len(out) // 2], max(out)

    mfma, mfma_max = time_it(lambda: binding.peak_mfma_bf16(4000, sink))
    buf = torch.empty(2, 1 << 28, device=dev, dtype=torch.float32)  # two 1 GiB halves
    buf.fill_(1.0)
    copy, copy_max = time_it(lambda: binding.peak_copy(buf[0], buf[1]))
    read, read_max = time_it(lambda: binding.peak_read(buf[0], sink))
    del buf
    return {"bf16_mfma_tflops": mfma / 1e12, "bf16_mfma_tflops_max": mfma_max / 1e12,
            "copy_gbps": copy / 1e9, "copy_gbps_max": copy_max / 1e9,
            "read_gbps": read / 1e9, "read_gbps_max": read_max / 1e9,
            "spec_bf16_mfma_tflops": metrics.MI355X_BF16_DENSE_TFLOPS, "spec_hbm_gbps": metrics.MI355X_HBM_GBPS,
            "note": "median of 5 launches of swa_peak_mfma_bf16 (MFMA-only loop, 8 waves per CU), swa_peak_copy "
                    "(1 GiB -> 1 GiB, read + write bytes) and swa_peak_read (1 GiB)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    choices=[w.name for w in W.WORKLOADS + W.EXTRA_WORKLOADS],
                    help="time this workload alone (default: the headline plus the suite)")
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
    by_name = {w.name: w for w in W.WORKLOADS + W.EXTRA_WORKLOADS}
    suite = args.workload is None
    head_name = HEADLINE if suite else args.workload

    # inputs first (host work), so the GPU measurements below run back to back
    head = Case(by_name[head_name], dev)
    others = [Case(by_name[n], dev) for n in SUITE] if suite else []
    torch.cuda.synchronize()

    peaks = measure_peaks(dev) if suite else None
    for c in others:
        c.timed(args.warmup, args.steps)
    head.timed(args.warmup, args.steps)
    spread = head.launch_spread()
    cold = head.cold_us(dev) if head.kind == "sparse" else None

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    r = head.result(peaks)
    line = {
        "metric": r["metric"], "value": r["value"], "unit": r["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": r["dtype"], "data": "synthetic (seeded generator, inputs resident in HBM)",
        "config": r["config"], "roofline": r["roofline"], "cpu_baseline": None,
    }
    line["launch_us"] = spread
    line["clock_ramp_ms"] = CLOCK_RAMP_MS
    if cold is not None:
        line["cold"] = {"us": cold, "value": head.work / (cold * 1e-6) / 1e9, "unit": r["unit"],
                        "note": "median of 5 launches, each after a 512 MiB device write that evicts the key table"}
    if suite:
        line["configs"] = {c.wl.name: c.result(peaks) for c in others}
        line["measured_peaks"] = peaks
        line["order"] = ("probes, then " + ", ".join(SUITE) + ", then the headline, each 50 ms of clock-ramp "
                         "steps + W warm-up + K timed steps back to back on the GPU; oracle baselines on the host "
                         "afterwards")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = head.cpu_baseline(10.0)
        for c in others:
            line["configs"][c.wl.name]["cpu_baseline"] = c.cpu_baseline(6.0)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
