#!/usr/bin/env python3
"""Benchmark of the sparse-attention backward on one MI355X.

One step = one sparse_attn_bwd call (every kernel of the backward: zero
fill, D preprocess, the row kernel with the gathers and five MFMA products,
dSinks, casts) over the MLA shared-KV token-sparse workload (B=1, S=8192,
64 heads, latent KV 576 with V = first 512, top-2048 per query), inputs
already resident in HBM.  O and lse come from the library's own forward,
outside the timed region.

Prints one JSON line: throughput in selected-KV TFLOP/s (sum over valid
(query, head, key) triples of 2 * (3 * d_qk + 2 * d_v) FLOP), the
roofline of the dominant kernel (timed on its own stream with HIP events
recorded by the library around it), and the fp64 oracle timed on a
bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from top_sparse_attention_gather_amd import binding as B  # noqa: E402
from top_sparse_attention_gather_amd import workloads as W  # noqa: E402

METRIC = "sparse-attn bwd TFLOP/s (selected-KV FLOPs) and % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the dominant kernel on the MLA 8K workload (the
# backward's main kernel in deterministic mode; "fwd": the forward) and on
# the 8K indexer workload ("idx": the per-token indexer kernel), from
# rocprofv3 FETCH_SIZE / WRITE_SIZE passes scaled by the same counters on a
# plain 1 GiB copy (`--copy-calibration`); valid only for the kernel source
# they were taken on (its SHA-256), else reported as null.
MEASURED_TRAFFIC = {
    ("mla_token_8k", "deterministic"): {
        "kernel_source": "top_sparse_attention_gather_amd/csrc/sa_bwd_mla.hip",
        "sha256": "d2c60c708983d71f54a451fb466db0cf0692e85f5dace0a3e6859f9564944931",
        "fetch_bytes": 8135253022, "write_bytes": 17517237920,
    },
    ("indexer_8k", "idx"): {
        "kernel_source": "top_sparse_attention_gather_amd/csrc/sa_indexer.hip",
        "sha256": "c011a9bac216114f734119104d90f9d5329e55a712b851d3cfe6e4cc5800d4d7",
        "fetch_bytes": 681986366, "write_bytes": 3894948128,
    },
    ("mla_token_8k", "fwd"): {
        "kernel_source": "top_sparse_attention_gather_amd/csrc/sa_fwd_rows.hip",
        "sha256": "b9e32a8b63797b9541203708503992ca55c0f67ede2e50dc2edeb25cee685ef6",
        "fetch_bytes": 2041776385, "write_bytes": 538968064,
    },
    ("nsa_block_gqa", "deterministic"): {
        "kernel_source": "top_sparse_attention_gather_amd/csrc/sa_bwd_blk.hip",
        "sha256": "532ff8dfd4707336ca19dc19d843505c0e62d394226ffa79b2c1eb1a0b2e7721",
        "fetch_bytes": 103939855, "write_bytes": 33554432,
    },
}


def measured_traffic(wl_name: str, mode: str):
    t = MEASURED_TRAFFIC.get((wl_name, mode))
    if t is None:
        return None
    with open(os.path.join(ROOT, t["kernel_source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["sha256"]:
            return None
    return t["fetch_bytes"] + t["write_bytes"]


def traffic_fields(wl_name: str, mode: str, off: bool = False):
    """roofline.traffic and where it comes from: a stored reading (not
    measured in this run) of two rocprofv3 counter passes, valid for the
    kernel source whose SHA-256 it was taken on, null otherwise."""
    t = MEASURED_TRAFFIC.get((wl_name, mode))
    val = None if off else measured_traffic(wl_name, mode)
    src = ("stored rocprofv3 FETCH_SIZE + WRITE_SIZE reading (copy-calibrated), taken on "
           f"{t['kernel_source']} sha256 {t['sha256'][:16]}; null when the source differs") if t else None
    return {"traffic": val,
            "traffic_unit": "bytes per launch (HBM fetch + write, copy-calibrated rocprofv3 counters)",
            "traffic_source": src if val is not None else (src and "not valid for this source or configuration")}


def host_info():
    """CPU model, logical CPU count and numpy's BLAS, for the CPU baseline."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpoolctl.threadpool_info()
                if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_info():
    """Compute units and peak engine clock of device 0 as HIP reports them
    (hipDeviceGetAttribute: hipDeviceAttributeMultiprocessorCount = 63,
    hipDeviceAttributeClockRate = 5, in kHz), and the dense bf16 MFMA peak
    they imply at 4 SIMDs per CU and 1024 FLOP per clock per SIMD."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        cus, khz = ctypes.c_int(0), ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0) or hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0):
            return None
    except OSError:
        return None
    return {"compute_units": cus.value, "max_sclk_mhz": khz.value / 1000.0,
            "bf16_peak_at_max_sclk_tflops": round(cus.value * 4 * 1024 * khz.value * 1e3 / 1e12, 1)}


def percentiles(ms):
    q = np.percentile(np.asarray(ms), [10, 50, 90])
    return {"p10": round(float(q[0]), 4), "median": round(float(q[1]), 4), "p90": round(float(q[2]), 4)}


def valid_pairs(wl: W.Workload, idx: np.ndarray) -> int:
    """Valid (token, kv head, key row) pairs from the generated indices,
    counted from the index lists (any negative slot is unused)."""
    if wl.select == W.SEL_TOKEN:
        return int((idx >= 0).sum())
    return W.expected_pair_count(wl)


def flops_per_pair(wl: W.Workload) -> int:
    return wl.group * 2 * (3 * wl.d_qk + 2 * wl.d_v)


def block_pairs(wl: W.Workload, idx: np.ndarray) -> int:
    """Valid (token, kv head, selected block) slots of a block-selection
    workload: the block starts inside the sequence and, causally, at or
    before the token."""
    cu = wl.cu_seqlens()
    tl = np.concatenate([np.arange(cu[b + 1] - cu[b]) for b in range(wl.batch)])[:, None, None]
    kv_len = np.concatenate([np.full(cu[b + 1] - cu[b], wl.seqlens[b]) for b in range(wl.batch)])[:, None, None]
    start = idx.astype(np.int64) * wl.block_size
    ok = (idx >= 0) & (start < kv_len) & (start <= tl)
    return int(ok.sum())


def main_kernel_roofline(wl: W.Workload, mode: str, idx: np.ndarray, flop: int, kern_ms: float):
    """Roofline of the dominant kernel: the MFMA row kernel (selected-KV
    FLOP / its time against the bf16 peak), or for block selection in
    deterministic mode the dQ pass over the selected blocks against HBM: its
    algorithmic HBM bytes are every input it needs read once (Q, dO, lse, D,
    the K/V rows, the indices) and dQ written once.  The selected blocks'
    rows are gathered again for every query (the gathered-row bytes, also
    reported with their rate), but the K/V of this shape is 4 MB and those
    re-reads come from L2, so HBM does not bound the kernel: the rate of its
    direct global->LDS block loads does."""
    if wl.select == W.SEL_BLOCK and mode == "deterministic":
        pairs = W.expected_pair_count(wl)
        T, H, Hkv = wl.total_q, wl.n_q_heads, wl.n_kv_heads
        nbytes = (T * H * (wl.d_qk + wl.d_v) * 2               # Q and dO read once
                  + T * H * 8                                   # lse and D
                  + wl.total_kv * Hkv * (wl.d_qk + wl.d_v) * 2  # K and V read once
                  + int(idx.size) * 4                           # indices
                  + T * H * wl.d_qk * 2)                        # dQ written
        gathered = pairs * (wl.d_qk + wl.d_v) * 2
        gbs = nbytes / (kern_ms * 1e-3) / 1e9
        return {"kernel": "blk_dq_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                "gathered_row_bytes": gathered,
                "gathered_row_rate_gbs": round(gathered / (kern_ms * 1e-3) / 1e9, 1),
                "block_pairs": block_pairs(wl, idx)}
    tf = flop / (kern_ms * 1e-3) / 1e12
    mla = wl.kv_shared and (wl.d_qk, wl.d_v) == (576, 512) and wl.select != W.SEL_BLOCK
    name = "mla_bwd_kernel" if mla else "bwd_rows_kernel"
    return {"kernel": name, "bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(inputs, wl, budget_s: float = 15.0, min_tokens: int = 8):
    """The fp64 oracle backward on the last query tokens (the longest
    rows), as many as fit the time budget; TFLOP/s of that sample."""
    from oracle import sparse_attn_oracle as O   # the oracle is only timed here
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        threads = len(os.sched_getaffinity(0))
    pb = O.Problem(inputs)
    T = wl.total_q
    done, flops, spent = 0, 0, 0.0
    chunk = min_tokens
    while spent < budget_s and done < T:
        toks = list(range(T - done - chunk, T - done))
        out, lse = O.sparse_fwd(pb, toks)
        Ob = torch.zeros(T, wl.n_q_heads, wl.d_v, dtype=torch.bfloat16)
        Lb = torch.zeros(T, wl.n_q_heads, dtype=torch.float32)
        ob, lb = O.round_fwd_outputs(out, lse)
        Ob[toks], Lb[toks] = ob, lb
        t0 = time.perf_counter()
        O.sparse_bwd(pb, Ob, Lb, tokens=toks)
        spent += time.perf_counter() - t0
        pairs = sum(pb.selection(t, g)[1].size for t in toks for g in range(wl.n_kv_heads))
        flops += pairs * flops_per_pair(wl)
        done += chunk
        chunk = min(2 * chunk, 64)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle sparse_bwd on the last {done} of {T} query tokens of {wl.name} "
                      f"({flops / 1e12:.3f} TFLOP in {spent:.1f} s, forward excluded)", **host_info()}


def indexer_cpu_baseline(inputs, wl, budget_s: float = 15.0, min_tokens: int = 8):
    """The fp64 oracle indexer gradient on the last tokens, as many as fit
    the time budget; TFLOP/s of that sample."""
    from oracle import sparse_attn_oracle as O   # the oracle is only timed here
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = wl.total_q
    idx = inputs["idx"].numpy()
    done, flops, spent, chunk = 0, 0, 0.0, min_tokens
    while spent < budget_s and done < T:
        toks = list(range(T - done - chunk, T - done))
        t0 = time.perf_counter()
        O.indexer_grad_kl(inputs, tokens=toks)
        spent += time.perf_counter() - t0
        flops += int((idx[toks] >= 0).sum()) * 6 * wl.n_q_heads * wl.d_qk
        done += chunk
        chunk = min(2 * chunk, 64)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle indexer_grad_kl on the last {done} of {T} query tokens of {wl.name} "
                      f"({flops / 1e12:.4f} TFLOP in {spent:.1f} s)", **host_info()}


def bench_indexer(args):
    """Sparse lightning-indexer gradient with the KL loss: one step = one
    sparse_attn_indexer_grad_kl call (CSR, the per-token kernel, the dK~
    reduction and cast, the loss sum).  FLOP: the three products S~ = q~K~^T,
    dq~ = dS~K~ and dK~ = dS~^T q~, 2 H d each per valid (token, row)."""
    wl = W.INDEXER_WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: generating inputs")
    inputs = W.make_indexer_inputs(wl, threads=16)
    idx = inputs["idx"].numpy()
    pairs = int((idx >= 0).sum())
    H, d, T, K = wl.n_q_heads, wl.d_qk, wl.total_q, wl.topk
    flop = pairs * 6 * H * d
    dev = B.indexer_device_tensors(inputs)
    desc = B.make_indexer_desc(wl)
    outputs = {"dq": torch.empty_like(dev["q"]), "dk": torch.empty_like(dev["k"]),
               "dweights": torch.empty((T, H), dtype=torch.float32, device="cuda"),
               "loss": torch.empty(1, dtype=torch.float32, device="cuda"),
               "loss_per_token": torch.empty(T, dtype=torch.float32, device="cuda")}
    ws = torch.empty(max(B.sparse_attn_indexer_grad_kl_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        B.sparse_attn_indexer_grad_kl(desc, dev, outputs, ws)
    torch.cuda.synchronize()
    ev = B.HipEvents(args.steps)
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    evict = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if args.evict_cache else None
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        if evict is not None:
            evict.fill_(float(i))
        calls[i][0].record(stream)
        B.sparse_attn_indexer_grad_kl(desc, dev, outputs, ws, stream=stream, events=ev.pairs[i])
        calls[i][1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in calls]
    ms = float(np.mean(call_ms)) if evict is not None else t_start.elapsed_time(t_stop) / args.steps
    kern_ms = float(np.mean([ev.elapsed_ms(i) for i in range(args.steps)]))
    ev.close()
    for k, v in outputs.items():
        if not torch.isfinite(v.float()).all():
            raise RuntimeError(f"non-finite values in {k}")
    tflops = flop / (ms * 1e-3) / 1e12
    # the per-token kernel's HBM bytes: q~, W, target, indices read once;
    # dq~, dW and the bf16 partial dK~ rows written (the gathered K~ rows,
    # 2 MB in all, are served from L2)
    nbytes = T * H * d * 2 + T * H * 4 + T * K * 8 + T * H * d * 2 + T * H * 4 + pairs * d * 2
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    ktf = flop / (kern_ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step, kernel {kern_ms:.3f} ms ({gbs:.0f} GB/s, {ktf:.1f} TFLOP/s)")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = indexer_cpu_baseline(inputs, wl, budget_s=args.cpu_budget)
    line = {
        "metric": "sparse lightning-indexer grad + KL loss TFLOP/s (selected-row FLOPs), 1 GPU",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.batch} S={wl.seqlens[0]} indexer heads={H} d={d} top-{K}",
                   "valid_pairs": pairs, "selected_row_tflop": round(flop / 1e12, 4),
                   "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "parallelism": "single GPU"},
        "timing": {"call_ms": percentiles(call_ms), "cache_evicted_between_calls": evict is not None,
                   "step_time_from": "per-call events" if evict is not None else "bracketed region / steps",
                   "device": device_info()},
        "roofline": {"kernel": "idx_grad_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                     "mfma_tflops": round(ktf, 2), **traffic_fields(wl.name, "idx"),
                     "kernel_ms": round(kern_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def workload_of(args) -> W.Workload:
    """The named workload with the command line's head, top-k and format
    overrides (named in the workload's name)."""
    wl = W.WORKLOADS[args.workload]
    over = {}
    if args.heads:
        over["n_q_heads"] = args.heads * wl.n_kv_heads
    if args.topk:
        over["topk"] = args.topk
    if args.dtype:
        over["dtype"] = args.dtype
    if over:
        wl = dataclasses.replace(wl, name=wl.name + "".join(f"+{k}={v}" for k, v in over.items()), **over)
    return wl


def fwd_flops_per_pair(wl: W.Workload) -> int:
    """S = q K^T and O = P V: 2 (d_qk + d_v) per head and selected row."""
    return wl.group * 2 * (wl.d_qk + wl.d_v)


def bench_forward(args):
    """Selected-attention forward (O and lse), the step before the backward:
    one step = one sparse_attn_fwd call, a single kernel launch, so the
    per-call events time that kernel."""
    wl = workload_of(args)
    log(f"[bench] workload {wl.name} (forward): generating inputs")
    inputs = W.make_inputs(wl, threads=16)
    idx = inputs["idx"].numpy()
    pairs = valid_pairs(wl, idx)
    flop = pairs * fwd_flops_per_pair(wl)
    dev = B.device_tensors(inputs)
    desc = B.make_desc(wl)
    stream = torch.cuda.current_stream()
    o, lse = B.sparse_attn_fwd(desc, dev, stream=stream)
    for _ in range(args.warmup):
        B.sparse_attn_fwd(desc, dev, o, lse, stream=stream)
    torch.cuda.synchronize()
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} forward steps")
    t_start.record(stream)
    for i in range(args.steps):
        calls[i][0].record(stream)
        B.sparse_attn_fwd(desc, dev, o, lse, stream=stream)
        calls[i][1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in calls]
    ms = t_start.elapsed_time(t_stop) / args.steps
    kern_ms = float(np.mean(call_ms))
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite values in o")
    tflops = flop / (ms * 1e-3) / 1e12
    kern_tflops = flop / (kern_ms * 1e-3) / 1e12
    log(f"[bench] forward {ms:.3f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import sparse_attn_oracle as O   # the oracle is only timed here
        try:
            import threadpoolctl
            threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or os.cpu_count()
        except Exception:
            threads = len(os.sched_getaffinity(0))
        pb = O.Problem(inputs)
        T = wl.total_q
        done, fl, spent, chunk = 0, 0, 0.0, 8
        while spent < args.cpu_budget and done < T:
            toks = list(range(T - done - chunk, T - done))
            t0 = time.perf_counter()
            O.sparse_fwd(pb, toks)
            spent += time.perf_counter() - t0
            fl += sum(pb.selection(t, g)[1].size for t in toks for g in range(wl.n_kv_heads)) * fwd_flops_per_pair(wl)
            done += chunk
            chunk = min(2 * chunk, 64)
        cpu = {"value": fl / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
               "sample": f"fp64 numpy oracle sparse_fwd on the last {done} of {T} query tokens of {wl.name} "
                         f"({fl / 1e12:.3f} TFLOP in {spent:.1f} s)", **host_info()}
    kernel = "fwd_mla_kernel" if (wl.d_qk, wl.d_v, wl.kv_shared) == (576, 512, True) \
        else "fwd_rows_kernel"
    line = {
        "metric": "sparse-attn fwd TFLOP/s (selected-KV FLOPs), 1 GPU",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} forward: B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
                               f"d_qk={wl.d_qk} d_v={wl.d_v} top-{wl.topk}",
                   "valid_pairs": pairs, "selected_kv_tflop": round(flop / 1e12, 4),
                   "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "parallelism": "single GPU"},
        "timing": {"call_ms": percentiles(call_ms), "step_time_from": "bracketed region / steps",
                   "device": device_info()},
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": round(kern_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     **traffic_fields(wl.name, "fwd", off=kernel != "fwd_mla_kernel"),
                     "kernel_ms": round(kern_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mla_token_8k",
                    choices=W.WORKLOAD_ORDER + list(W.INDEXER_WORKLOADS))
    ap.add_argument("--op", default="bwd", choices=["bwd", "fwd"],
                    help="bwd: the backward (the default line); fwd: the selected-attention forward alone")
    ap.add_argument("--heads", type=int, default=0,
                    help="override the workload's query heads per kv head (sweeps off the 64-head shape)")
    ap.add_argument("--topk", type=int, default=0, help="override the workload's index slots per row")
    ap.add_argument("--dtype", default="", choices=["", "bf16", "fp16"], help="override the 16-bit input format")
    ap.add_argument("--dkv-mode", default="deterministic", choices=["atomic", "deterministic", "atomic_xcd"],
                    help="dK/dV reduction: fp32 atomics, the deterministic key-major pass, or (shared-KV MLA "
                         "shapes) fp32 atomics into one accumulator copy per XCD")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--softmax-l1", action="store_true",
                    help="also produce the softmax L1-norm side outputs in every timed call")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--evict-cache", action="store_true",
                    help="write 1 GiB before every timed call (evicts the 256 MB Infinity Cache); the step time "
                         "is then the mean of the per-call events")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed steps, this many calls each preceded by a 1 GiB eviction write, "
                         "reported as timing.cold_cache (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (read 1 GiB, write 1 GiB): the known-size kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (see the design notes on "
              "sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return

    if args.workload in W.INDEXER_WORKLOADS:
        bench_indexer(args)
        return
    if args.op == "fwd":
        bench_forward(args)
        return
    wl = workload_of(args)
    mode = {"atomic": B.DKV_ATOMIC, "deterministic": B.DKV_DETERMINISTIC, "atomic_xcd": B.DKV_ATOMIC_XCD}[args.dkv_mode]
    log(f"[bench] workload {wl.name}: generating inputs")
    inputs = W.make_inputs(wl, threads=16)
    idx = inputs["idx"].numpy()
    pairs = valid_pairs(wl, idx)
    flop = pairs * flops_per_pair(wl)
    dev = B.device_tensors(inputs)
    desc = B.make_desc(wl, mode, softmax_l1=int(args.softmax_l1))
    log("[bench] forward (inputs O, lse)")
    dev["o"], dev["lse"] = B.sparse_attn_fwd(desc, dev)
    outputs = B.alloc_bwd_outputs(desc, dev)
    ws = torch.empty(max(B.sparse_attn_bwd_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        B.sparse_attn_bwd(desc, dev, outputs, ws)
    torch.cuda.synchronize()

    ev = B.HipEvents(args.steps)
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    # one event pair around every call, on the stream the library launches on
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    evict = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if args.evict_cache else None
    log(f"[bench] timing {args.steps} steps" + (" (Infinity Cache evicted before each call)" if evict is not None else ""))
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        if evict is not None:
            evict.fill_(float(i))            # 1 GiB written between calls, outside the per-call events
        calls[i][0].record(stream)
        B.sparse_attn_bwd(desc, dev, outputs, ws, stream=stream, events=ev.pairs[i])
        calls[i][1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in calls]
    total_ms = t_start.elapsed_time(t_stop)
    # with eviction the bracketed region also holds the eviction writes, so
    # the step time is the mean of the per-call events
    ms = float(np.mean(call_ms)) if evict is not None else total_ms / args.steps
    kern_ms = float(np.mean([ev.elapsed_ms(i) for i in range(args.steps)]))
    ev.close()
    for k, v in outputs.items():
        if not torch.isfinite(v.float()).all():
            raise RuntimeError(f"non-finite values in {k}")

    tflops = flop / (ms * 1e-3) / 1e12
    kern_tflops = flop / (kern_ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step, main kernel {kern_ms:.3f} ms, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")

    # the same call with a cold cache beside the warm figure: 1 GiB written
    # before each call (outside its events) evicts the 256 MB Infinity Cache
    cold = None
    if evict is None and args.cold_steps > 0:
        big = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            big.fill_(float(i))
            cold_ev[i][0].record(stream)
            B.sparse_attn_bwd(desc, dev, outputs, ws, stream=stream)
            cold_ev[i][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = [a.elapsed_time(b) for a, b in cold_ev]
        del big
        cold = {"calls": args.cold_steps, "call_ms": percentiles(cold_ms),
                "value": round(flop / (float(np.mean(cold_ms)) * 1e-3) / 1e12, 3)}
        log(f"[bench] cold cache: {float(np.mean(cold_ms)):.3f} ms/call")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(inputs, wl, budget_s=args.cpu_budget)
        log(f"[bench] cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.batch} S={wl.seqlens[0] if wl.batch == 1 else list(wl.seqlens)} "
                        f"Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} d_qk={wl.d_qk} d_v={wl.d_v} "
                        f"{'shared-KV ' if wl.kv_shared else ''}top-{wl.topk}",
            "dkv_mode": args.dkv_mode,
            "softmax_l1_outputs": bool(args.softmax_l1),
            "valid_pairs": pairs,
            "selected_kv_tflop": round(flop / 1e12, 4),
            "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "parallelism": "single GPU",
        },
        "timing": {"call_ms": percentiles(call_ms), "cache_evicted_between_calls": evict is not None,
                   "step_time_from": "per-call events" if evict is not None else "bracketed region / steps",
                   "cold_cache": cold, "device": device_info()},
        "roofline": dict(main_kernel_roofline(wl, args.dkv_mode, idx, flop, kern_ms), **{
            # the stored counter readings are of the kernel without the L1-norm sums
            **traffic_fields(wl.name, args.dkv_mode, off=args.softmax_l1),
            "kernel_ms": round(kern_ms, 4),
        }),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
