#!/usr/bin/env python3
"""Throughput of the reranker hot path on one MI355X: scored query-passage pairs/s.

A step is one pass of the whole hot path over one synthetic batch with every
input already resident in HBM: pair layout, chunk pooling, the cross K/V of
every layer, the merged-attention decoder stack and the yes/no score.  The
default workload is the Small-shaped stack (32 queries x 100 passages, 26
layers, H=1152, 4 query heads / 1 KV head, head dim 256, bf16 storage with fp32
accumulation).  Every libkalm call of the timed steps is bracketed with HIP
events on the launch stream, which gives each kernel's average duration and,
with its algorithmic work, its roofline fraction.  The CPU oracle is timed on a
bounded seeded sample of the same workload on the host cores.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import contextlib
import json
import math
import os
import sys
import time
from collections import defaultdict

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop/byte where the two roofs meet

# HBM bytes per launch from two rocprofv3 --pmc runs of this bench at its
# default workload (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
# by what the same counter reads for a plain 1 GiB device copy (bench.py
# --copy-probe: FETCH_SIZE reads half the bytes copied, WRITE_SIZE all of
# them, so the factors are 2.0 and 1.0).  Keyed by kernel; "src" is the
# sha256 of the source file the kernel was built from when the counters were
# taken -- after any change to that file the traffic is reported as null.
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
MEASURED_TRAFFIC = {
    # profiles/hbm_traffic_small_stack26_bf16.md (the QKV figures are the mean over the full-height
    # launches only; the same kernel symbol also runs the last layer's K/V projection)
    "qkv_linear": {"src": "25b4c172737f9f7a78d46b8f8ebd2509231b9bbf8b505cdbf3421072b3dd7c7b", "fetch_kib": 1880075.5, "write_kib": 2688306.2},
    "o_linear": {"src": "25b4c172737f9f7a78d46b8f8ebd2509231b9bbf8b505cdbf3421072b3dd7c7b", "fetch_kib": 3114048.0, "write_kib": 6544855.2},
    "merged_attn": {"src": "7789502f81c8b83a4def65d09a3941259f87406efa97af929c8fe8edf79695fd", "fetch_kib": 1348960.8, "write_kib": 1792200.0},
}
# the source files each kernel is built from (headers included); their joint
# sha256 keys the stored counter values
KERNEL_SRC = {"o_linear": ("gemm.hip", "kalm_common.h"), "qkv_linear": ("gemm.hip", "kalm_common.h"),
              "cross_kv": ("gemm.hip", "kalm_common.h"),
              "merged_attn": ("attn.hip", "attn_bf16.h", "kalm_common.h"),
              "chunk_pool": ("pool.hip", "kalm_common.h"), "gather_rows": ("rows.hip", "kalm_common.h")}


def source_sha(kernel):
    """sha256 over the source files a kernel is built from (None if unknown)."""
    import hashlib
    srcs = KERNEL_SRC.get(kernel)
    if not srcs:
        return None
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, "encoder_decoder_document_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """Counter-measured HBM bytes per launch, or None when stale or not measured."""
    m = MEASURED_TRAFFIC.get(kernel)
    if not m or m["src"] != source_sha(kernel):
        return None
    return m["fetch_kib"] * 1024 * FETCH_FACTOR + m["write_kib"] * 1024 * WRITE_FACTOR
METRIC = "scored query-passage pairs/s (1 GPU) + merged-attn MFMA util % / pool HBM GB/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="small_stack26_bf16")
    ap.add_argument("--chunk", type=int, default=None,
                    help="pooling granularity in tokens (Matryoshka variants); default: the workload's (4)")
    ap.add_argument("--no-prune", action="store_true",
                    help="compute every row of the first and last layers (no shared / final-row shortcut)")
    ap.add_argument("--no-reuse-self", action="store_true",
                    help="first layer in one merged pass per pair instead of each query's self part once")
    ap.add_argument("--mlp-dim", type=int, default=None,
                    help="model-shaped layers (RMSNorm, RoPE, gated-GELU MLP of this width) around the attention")
    ap.add_argument("--split-kv", action="store_true",
                    help="one-layer stacks: each pair's cross keys in shares over several workgroups")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as a HIP graph (per-kernel times from the eager "
                         "warm-up steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--no-pool-long", action="store_true", help="skip the pooling measurement at the 1024x2560 shape")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (Nano single layer, Nano stack, Long/wide) measured after the "
                         "headline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates the HBM byte counters)")
    return ap.parse_args()


class EventRec:
    """Records a start/stop HIP event pair on the current stream around each call."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = defaultdict(list)
        self.on = True

    @contextlib.contextmanager
    def __call__(self, name):
        if not self.on:
            yield
            return
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        yield
        e.record()
        self.ev[name].append((s, e))

    def durations_ms(self):
        self.torch.cuda.synchronize()
        return {k: [s.elapsed_time(e) for s, e in v] for k, v in self.ev.items()}


def model_work(inp, sh, work, single=False):
    """Work per launch of the model-shaped layer's extra calls (RMSNorm, RoPE,
    gated MLP in passes of at most MLP_ROWS rows, final norm)."""
    from encoder_decoder_document_amd.stack import MLP_ROWS
    I = int(inp["model"]["mlp_dim"])
    H, nq, nkv, d = sh.H, sh.nq, sh.nkv, sh.d
    e = 2 if sh.dtype == "bf16" else 4
    lq = np.asarray(inp["lq"], dtype=np.int64)
    U, P = int(lq.sum()), sh.pairs
    rows = sh.n_docs * U

    def norm(m):
        return dict(flops=3.0 * m * H, bytes=float(m * H * (4 + e) + H * e))

    def rope(m, heads):
        return dict(flops=6.0 * m * heads * d, bytes=float(2 * m * heads * d * e))

    def mlp(m, tag):
        n_pass = -(-m // MLP_ROWS)
        c = m / n_pass  # rows per pass (average)
        work.update({
            "mlp_norm" + tag: norm(c),
            "mlp_gate_up" + tag: dict(flops=2.0 * c * H * 2 * I, bytes=float(c * H * e + 2 * I * H * e + c * 2 * I * e)),
            "mlp_act" + tag: dict(flops=8.0 * c * I, bytes=float(c * 3 * I * e)),
            "mlp_down" + tag: dict(flops=2.0 * c * I * H, bytes=float(c * I * e + H * I * e + c * H * 8)),
            # fused gate/up projection and activation: only the activation leaves the CU
            "mlp_gate_up_act" + tag: dict(flops=2.0 * c * H * 2 * I + 8.0 * c * I,
                                          bytes=float(c * H * e + 2 * I * H * e + c * I * e)),
        })

    work.update({"attn_norm": norm(rows), "attn_norm_first": norm(U), "attn_norm_last": norm(P),
                 "rope_q": rope(rows, nq), "rope_k": rope(rows, nkv), "rope_q_first": rope(U, nq),
                 "rope_k_first": rope(U, nkv), "rope_q_last": rope(P, nq),
                 "final_norm": dict(flops=3.0 * P * H, bytes=float(P * H * 8 + H * e))})
    if not single:
        mlp(rows, "")
    mlp(P, "_last")
    return work


def work_model(inp, sh, single=False):
    """Algorithmic work per launch of each recorded call (flops and bytes).

    Names follow the step: the full-size projections and attention of the
    middle layers, the first layer (Q/K/V once per query row, attention over
    shared rows) and the last layer (final rows only)."""
    D, T, H, nq, nkv, d = sh.n_docs, sh.T, sh.H, sh.nq, sh.nkv, sh.d
    lq = np.asarray(inp["lq"], dtype=np.int64)
    dl = np.asarray(inp["doc_len"], dtype=np.int64)
    C = -(-dl // sh.chunk)                    # valid chunks per passage (right padding)
    Cmax = -(-T // sh.chunk)
    e = 2 if sh.dtype == "bf16" else 4
    rows = int(D * lq.sum())                  # decoder rows of all pairs
    U = int(lq.sum())                         # decoder rows of the queries themselves
    P = sh.pairs
    qd, kv = nq * d, nkv * d
    nqkv = qd + 2 * kv
    self_keys = int((lq * (lq + 1) // 2).sum()) * D     # causal (row, key) pairs over all pairs
    cross_keys = int(lq.sum()) * int(C.sum())            # (row, chunk) pairs over all pairs
    attn_flops = 4 * nq * d * (self_keys + cross_keys)
    self_bytes = 2 * rows * kv * e                       # self K and V, once
    cross_bytes = 2 * int(C.sum()) * kv * e
    last_flops = 4 * nq * d * (int(lq.sum()) * D + len(lq) * int(C.sum()))  # final row: Lq self + C cross keys

    def linear(M, K, N, out_bytes):
        return dict(flops=2.0 * M * K * N, bytes=float(M * K * e + N * K * e + out_bytes))

    # every layer's cross K/V in one launch: the valid chunk rows of all
    # passages projected by each layer's weights; pooled rows read once, the
    # stacked weights once, every output row (padded ones written as 0) once
    L = len(inp["layers"])
    cross_kv = dict(flops=2.0 * L * int(C.sum()) * H * 2 * kv,
                    bytes=float(D * Cmax * H * e + L * 2 * kv * H * e + D * Cmax * L * 2 * kv * e))

    if single:
        # one pruned layer: the queries' own rows and every pair's final row only
        nQ = len(lq)
        return {
            "qkv_linear_first": linear(U, H, nqkv, U * nqkv * e),
            "self_attn_first": dict(flops=float(4 * nq * d * self_keys // D),
                                    bytes=float(U * qd * e + 2 * U * kv * e + U * qd * 4 + U * nq * 4)),
            "merged_attn_first_resume": dict(flops=float(4 * nq * d * nQ * int(C.sum())),
                                             bytes=float(nQ * qd * e + nQ * (qd + nq) * 4 + cross_bytes
                                                         + P * qd * e)),
            "merged_attn_first": dict(flops=float(last_flops),
                                      bytes=float(nQ * qd * e + 2 * U * kv * e + cross_bytes + P * qd * e)),
            # split-KV: the shares' fp32 partials are written and read back by the merge
            "merged_attn_first_split": dict(flops=float(4 * nq * d * nQ * int(C.sum())),
                                            bytes=float(nQ * qd * e + nQ * (qd + nq) * 4 + cross_bytes
                                                        + P * qd * e)),
            "o_linear_last": linear(P, qd, H, P * H * 8),
            "cross_kv": cross_kv,
            "chunk_pool": dict(flops=0.0, bytes=float(int(dl.sum()) * H * e + D * Cmax * H * e + D * T + D * Cmax
                                                      + 4 * D)),
            "gather_query_rows": dict(flops=0.0, bytes=float(U * H * (4 + 4 + 2))),
            "gather_final_rows": dict(flops=0.0, bytes=float(P * H * (4 + 4))),
        }

    return {
        "merged_attn": dict(flops=float(attn_flops), bytes=float(2 * rows * qd * e + self_bytes + cross_bytes)),
        "merged_attn_first": dict(flops=float(attn_flops),
                                  bytes=float(U * qd * e + rows * qd * e + 2 * U * kv * e + cross_bytes)),
        # first layer split at the self/cross boundary: each query's causal self
        # part once (fp32 output and lse), then every pair's cross part resumed
        # from it
        "self_attn_first": dict(flops=float(4 * nq * d * self_keys // D),
                                bytes=float(U * qd * e + 2 * U * kv * e + U * qd * 4 + U * nq * 4)),
        "merged_attn_first_resume": dict(flops=float(4 * nq * d * cross_keys),
                                         bytes=float(U * qd * e + U * qd * 4 + U * nq * 4 + cross_bytes
                                                     + rows * qd * e)),
        "merged_attn_last": dict(flops=float(last_flops), bytes=float(2 * P * qd * e + self_bytes + cross_bytes)),
        "qkv_linear": linear(rows, H, nqkv, rows * nqkv * e),
        "qkv_linear_first": linear(U, H, nqkv, U * nqkv * e),
        "kv_linear_last": linear(rows, H, 2 * kv, rows * 2 * kv * e),
        "q_linear_last": linear(P, H, qd, P * qd * e),
        # residual update: read and write the fp32 stream, write its bf16 copy
        "o_linear": linear(rows, qd, H, rows * H * (4 + 4 + (2 if e == 2 else 0))),
        # first layer: the residual source is each query's first hidden rows, read once
        "o_linear_first": linear(rows, qd, H, U * H * 4 + rows * H * (4 + (2 if e == 2 else 0))),
        "o_linear_last": linear(P, qd, H, P * H * 8),
        "cross_kv": cross_kv,
        "chunk_pool": dict(flops=0.0, bytes=float(int(dl.sum()) * H * e + D * Cmax * H * e + D * T + D * Cmax + 4 * D)),
        # residual start: the queries' first hidden states read once, every pair row written fp32 + bf16
        "gather_rows": dict(flops=0.0, bytes=float(U * H * 4 + rows * H * (4 + (2 if e == 2 else 0)))),
        "gather_query_rows": dict(flops=0.0, bytes=float(U * H * (4 + 4 + 2))),
        "gather_final_rows": dict(flops=0.0, bytes=float(P * H * (4 + 4 + 2))),
    }


def attn_summary(kernels, work, sh):
    """All merged-attention launches of a step together (every row mode, and
    the self and resumed parts of a split first layer): useful
    flops and algorithmic bytes over their summed time."""
    names = [k for k in kernels if (k.startswith("merged_attn") or k.startswith("self_attn")) and k in work]
    t = sum(kernels[k]["total_ms_per_step"] for k in names) * 1e-3
    if not names or t <= 0:
        return None
    fl = sum(work[k]["flops"] * kernels[k]["launches_per_step"] for k in names)
    by = sum(work[k]["bytes"] * kernels[k]["launches_per_step"] for k in names)
    peak = PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS
    return {"launches_per_step": sum(kernels[k]["launches_per_step"] for k in names), "ms_per_step": t * 1e3,
            "tflops": fl / t / 1e12, "mfma_frac": fl / t / 1e12 / peak, "gbs": by / t / 1e9,
            "hbm_frac": by / t / 1e9 / PEAK_HBM_GBS}


def cpu_baseline(inp, sh, budget_s):
    import threadpoolctl
    import oracle
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
    rng = np.random.default_rng(0)
    order = rng.permutation(sh.pairs)
    done = 0
    t0 = time.perf_counter()
    for p in order:
        oracle.stack_scores(inp, pairs=[int(p)], mode="mirror")
        done += 1
        if time.perf_counter() - t0 >= budget_s and done >= 2:
            break
    el = time.perf_counter() - t0
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": done / el, "unit": "pairs/s", "cores": int(cores), "kind": "oracle",
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
            "sample": f"{done} seeded-random pairs of the same workload, all {sh.n_layers} layers each, "
                      f"pooling + cross K/V per pair, fp64 numpy (mirror mode), {el:.1f} s",
            "blas": ";".join(sorted({f"{i.get('internal_api')}:{i.get('num_threads')}" for i in info}))}


def pool_long(torch, ops, reps=20):
    """Pooling at the 100 x 1024-token x 2560 shape (every chunk full)."""
    D, T, H = 100, 1024, 2560
    g = torch.Generator(device="cuda").manual_seed(1234)
    x = torch.randn(D, T, H, device="cuda", dtype=torch.bfloat16, generator=g)
    m = torch.ones(D, T, dtype=torch.uint8, device="cuda")
    C = T // 4
    out = (torch.empty(D, C, H, dtype=torch.bfloat16, device="cuda"),
           torch.empty(D, C, dtype=torch.uint8, device="cuda"), torch.empty(D, dtype=torch.int32, device="cuda"))
    for _ in range(3):
        ops.kalm_chunk_pool(x, m, 4, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record()
        ops.kalm_chunk_pool(x, m, 4, out=out)
        e.record()
    torch.cuda.synchronize()
    ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    by = D * T * H * 2 + D * C * H * 2 + D * T + D * C + 4 * D
    del x, out
    return {"shape": "100 x 1024 tokens x 2560 bf16, chunk 4", "avg_us": ms * 1e3,
            "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": by}


def kernel_table(dur, work, steps, sh):
    """Per recorded call: launches per step, average duration, and against its
    algorithmic work the achieved rate and roofline fractions."""
    kernels = {}
    for k, v in dur.items():
        n_per = len(v) / steps
        avg_us = float(np.mean(v)) * 1e3
        ent = {"launches_per_step": n_per, "avg_us": avg_us, "total_ms_per_step": float(np.sum(v)) / steps}
        if k in work:
            w = work[k]
            if w["flops"] > 0:
                ent["tflops"] = w["flops"] / (avg_us * 1e-6) / 1e12
                ent["mfma_frac"] = ent["tflops"] / (PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS)
            ent["gbs"] = w["bytes"] / (avg_us * 1e-6) / 1e9
            ent["hbm_frac"] = ent["gbs"] / PEAK_HBM_GBS
        kernels[k] = ent
    return kernels


def other_workload(torch, stack, synth, idx, steps, warmup, graph):
    """Pairs/s of one more workload (eager steps, and replays of the step
    captured as a HIP graph when ``graph``), with its merged attention's
    useful-flop rate and the per-kernel split."""
    sh = synth.SHAPES[idx]
    print(f"[bench] other workload {sh.name}: generating", file=sys.stderr, flush=True)
    inp = synth.make_inputs(idx, nan_padding=False)
    b = stack.upload(inp)
    for _ in range(warmup):
        stack.step(b)
    torch.cuda.synchronize()
    # pairs/s from plain eager steps; per-kernel times from as many more steps
    # with HIP events around each call (recording them costs host time that
    # would count against the microsecond steps of the small workloads)
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step(b)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    rec = EventRec(torch)
    for _ in range(steps):
        stack.step(b, rec=rec)
    single = sh.n_layers == 1
    kernels = kernel_table(rec.durations_ms(), work_model(inp, sh, single=single), steps, sh)
    ent = {"workload": sh.name, "queries": sh.n_queries, "docs": sh.n_docs, "pairs": sh.pairs,
           "layers": sh.n_layers, "hidden": sh.H, "q_heads": sh.nq, "kv_heads": sh.nkv, "head_dim": sh.d,
           "steps": steps, "warmup": warmup, "ms_per_step": el * 1e3, "value": sh.pairs / el, "unit": "pairs/s",
           "merged_attn": attn_summary(kernels, work_model(inp, sh, single=single), sh),
           "kernels": {k: {kk: round(vv, 6) if isinstance(vv, float) else vv for kk, vv in v.items()}
                       for k, v in kernels.items()}}
    if graph:
        g = stack.StepGraph(b)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        n = max(steps, 20)
        t0 = time.perf_counter()
        for _ in range(n):
            g.replay()
        torch.cuda.synchronize()
        gl = (time.perf_counter() - t0) / n
        ent["graph"] = {"replays": n, "ms_per_step": gl * 1e3, "value": sh.pairs / gl, "unit": "pairs/s"}
        del g
    print(f"[bench] other workload {sh.name}: {el * 1e3:.3f} ms/step, {sh.pairs / el:.1f} pairs/s",
          file=sys.stderr, flush=True)
    del b
    torch.cuda.empty_cache()
    return ent


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would run its own "
              "passage shard independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read_per_launch": src.numel() * 4,
                          "copy_probe_bytes_written_per_launch": dst.numel() * 4, "launches": 5}), flush=True)
        return
    from encoder_decoder_document_amd import ops, stack, synth

    names = [s.name for s in synth.SHAPES]
    if a.workload not in names:
        sys.exit(f"unknown workload {a.workload}; one of {names}")
    idx = names.index(a.workload)
    sh = synth.SHAPES[idx]
    if a.chunk is not None:
        import dataclasses
        sh = dataclasses.replace(sh, chunk=a.chunk)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU (libkalm has no CPU fallback)")
    if ops.device_check() != ops.KALM_OK:
        sys.exit(ops.load().kalm_last_error().decode())
    print(f"[bench] generating {sh.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(idx, nan_padding=False, shape=sh, mlp_dim=a.mlp_dim)
    b = stack.upload(inp)
    torch.cuda.synchronize()
    print(f"[bench] uploaded: rows={b.rows} pairs={b.P}; warmup {a.warmup}", file=sys.stderr, flush=True)
    rec = EventRec(torch)
    rec.on = False
    for _ in range(a.warmup):
        stack.step(b, rec=rec, prune=not a.no_prune, reuse_self=not a.no_reuse_self, split_kv=a.split_kv)
    torch.cuda.synchronize()
    rec.on = True
    t0 = time.perf_counter()
    for i in range(a.steps):
        stack.step(b, rec=rec, prune=not a.no_prune, reuse_self=not a.no_reuse_self, split_kv=a.split_kv)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / a.steps * 1e3
    pairs_s = sh.pairs / (el / a.steps)
    print(f"[bench] {a.steps} steps: {ms_step:.2f} ms/step, {pairs_s:.1f} pairs/s", file=sys.stderr, flush=True)
    eager_ms = ms_step
    # warm cache: the passages' pooled vectors and cross K/V stay resident from
    # the steps above (the pages cache the passage encodings), so a query batch
    # costs the decoder and the readout only
    for _ in range(max(1, a.warmup)):
        stack.decoder(b, prune=not a.no_prune, reuse_self=not a.no_reuse_self, split_kv=a.split_kv)
        stack.score(b, prune=not a.no_prune)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        stack.decoder(b, prune=not a.no_prune, reuse_self=not a.no_reuse_self, split_kv=a.split_kv)
        stack.score(b, prune=not a.no_prune)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) / a.steps * 1e3
    print(f"[bench] warm cache (decoder + score): {warm_ms:.2f} ms/step", file=sys.stderr, flush=True)
    if a.graph:
        # the same step captured once as a HIP graph; the timed steps are replays
        g = stack.StepGraph(b, prune=not a.no_prune, reuse_self=not a.no_reuse_self, split_kv=a.split_kv)
        for _ in range(a.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        ms_step = el / a.steps * 1e3
        pairs_s = sh.pairs / (el / a.steps)
        print(f"[bench] {a.steps} graph replays: {ms_step:.3f} ms/step, {pairs_s:.1f} pairs/s", file=sys.stderr,
              flush=True)

    dur = rec.durations_ms()
    single = not a.no_prune and sh.n_layers == 1
    work = work_model(inp, sh, single=single)
    if inp.get("model"):
        model_work(inp, sh, work, single=single)
    kernels = kernel_table(dur, work, a.steps, sh)
    for k, ent in kernels.items():
        tb = traffic_bytes(k)
        if tb is not None:
            ent["hbm_traffic_bytes"] = tb
            ent["traffic_over_algorithmic"] = tb / work[k]["bytes"] if k in work else None
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k]["total_ms_per_step"])
    w = work[dom]
    ai = w["flops"] / w["bytes"] if w["bytes"] else float("inf")
    if w["flops"] > 0 and ai >= RIDGE:
        peak = PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["tflops"], "peak": peak,
                "unit": "TFLOP/s", "frac": kernels[dom]["tflops"] / peak}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": kernels[dom]["gbs"] / PEAK_HBM_GBS}
    roof.update({"traffic": traffic_bytes(dom), "algorithmic_flops_per_launch": w["flops"],
                 "algorithmic_bytes_per_launch": w["bytes"], "arith_intensity": ai, "avg_us": kernels[dom]["avg_us"],
                 # the same launch against the other roof (its flops against the MFMA peak, or its bytes
                 # against the HBM peak)
                 "other_roof": ({"bound": "mfma", "frac": kernels[dom].get("mfma_frac")} if roof["bound"] == "hbm"
                                else {"bound": "hbm", "frac": kernels[dom].get("hbm_frac")})})
    out = {
        "metric": METRIC, "value": pairs_s, "unit": "pairs/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) encoder states and first hidden states, N(0,0.02) weights)",
        "config": {"workload": sh.name, "queries": sh.n_queries, "docs": sh.n_docs, "pairs": sh.pairs,
                   "layers": sh.n_layers, "hidden": sh.H, "q_heads": sh.nq, "kv_heads": sh.nkv, "head_dim": sh.d,
                   "decoder_len": list(sh.lq), "passage_len": list(sh.doc_len), "chunk": sh.chunk,
                   "decoder_rows": b.rows, "pruned_first_last_layer": not a.no_prune,
                   "first_layer_self_once_per_query": not a.no_prune and not a.no_reuse_self,
                   "hip_graph": a.graph, "eager_ms_per_step": eager_ms,
                   "layer": ("model-shaped (RMSNorm, RoPE, gated-GELU MLP %d)" % a.mlp_dim) if a.mlp_dim
                   else "merged attention + projections",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "merged_attn": attn_summary(kernels, work, sh),
        "warm_cache": {"ms_per_step": warm_ms, "value": sh.pairs / (warm_ms * 1e-3), "unit": "pairs/s",
                       "what": "decoder + readout with the passages' pooled vectors and cross K/V resident "
                               "(eager launches)"},
        "kernels": kernels,
    }
    if not a.no_pool_long:
        out["pool_long"] = pool_long(torch, ops)
    del b
    torch.cuda.empty_cache()
    if not a.no_others and a.workload == "small_stack26_bf16" and a.chunk is None and not a.mlp_dim:
        # the other workloads, each timed on its own after the headline: the
        # one-layer and the Nano stack also as HIP-graph replays (their
        # kernels run for microseconds), Long/wide with few steps (4 s each)
        out["others"] = [other_workload(torch, stack, synth, 1, 20, 3, True),
                         other_workload(torch, stack, synth, 2, 10, 2, True),
                         other_workload(torch, stack, synth, 4, 2, 1, False)]
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, sh, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
