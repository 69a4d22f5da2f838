"""Host-side checks of bench.py's accounting (no GPU).

The roofline line divides the algorithmic work of one launch by its measured
duration, so the per-launch work is pinned here against counts made a
different way: the attention's visible (row, key) pairs by walking every pair,
the projections' bytes and flops from their operand shapes.  The stored
counter traffic must go stale when the kernel source changes, and a request
for several GPUs must stop with a message instead of running.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from encoder_decoder_document_amd import synth  # noqa: E402


def _visible_pairs(inp):
    """(self, cross) visible (decoder row, key) pairs over every pair, by walking them."""
    sh = inp["shape"]
    lq = np.asarray(inp["lq"])
    C = -(-np.asarray(inp["doc_len"]) // sh.chunk)
    n_self = n_cross = 0
    for q in range(sh.n_queries):
        for dd in range(sh.n_docs):
            for i in range(int(lq[q])):
                n_self += i + 1          # causal: row i sees self keys 0..i
                n_cross += int(C[dd])    # and every valid chunk of its passage
    return n_self, n_cross


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_work_model_matches_brute_force_counts(idx):
    inp = synth.make_inputs(idx)
    sh = inp["shape"]
    wm = bench.work_model(inp, sh)
    e = 2 if sh.dtype == "bf16" else 4
    nq, nkv, d, H = sh.nq, sh.nkv, sh.d, sh.H
    lq = np.asarray(inp["lq"])
    rows = int(sh.n_docs * lq.sum())
    n_self, n_cross = _visible_pairs(inp)
    # every visible (row, key) pair costs a d-long dot product and a d-long
    # weighted sum per query head: 2 d + 2 d flops
    assert wm["merged_attn"]["flops"] == 4 * nq * d * (n_self + n_cross)
    # Q read + O written per row; self K/V per row; cross K/V per valid chunk
    C = -(-np.asarray(inp["doc_len"]) // sh.chunk)
    assert wm["merged_attn"]["bytes"] == (2 * rows * nq * d + 2 * rows * nkv * d + 2 * int(C.sum()) * nkv * d) * e
    n_qkv = nq * d + 2 * nkv * d
    assert wm["qkv_linear"]["flops"] == 2 * rows * H * n_qkv
    assert wm["qkv_linear"]["bytes"] == (rows * H + n_qkv * H + rows * n_qkv) * e
    # residual update: O and the weights read, the fp32 stream read and
    # written, its bf16 copy written (bf16 workloads)
    copy = 2 if e == 2 else 0
    assert wm["o_linear"]["flops"] == 2 * rows * nq * d * H
    assert wm["o_linear"]["bytes"] == rows * nq * d * e + H * nq * d * e + rows * H * (4 + 4 + copy)


def test_single_layer_model_counts_final_rows_only():
    inp = synth.make_inputs(1)
    sh = inp["shape"]
    wm = bench.work_model(inp, sh, single=True)
    lq = np.asarray(inp["lq"])
    C = -(-np.asarray(inp["doc_len"]) // sh.chunk)
    # one final row per pair: Lq self keys + its passage's chunks
    final_pairs = sum(int(lq[q]) + int(C[dd]) for q in range(sh.n_queries) for dd in range(sh.n_docs))
    assert wm["merged_attn_first"]["flops"] == 4 * sh.nq * sh.d * final_pairs
    assert wm["o_linear_last"]["flops"] == 2 * sh.pairs * sh.nq * sh.d * sh.H


def test_counter_traffic_goes_stale_with_the_source(monkeypatch):
    import hashlib
    for k in bench.KERNEL_SRC:
        h = hashlib.sha256()
        for src in bench.KERNEL_SRC[k]:
            h.update(open(os.path.join(ROOT, "encoder_decoder_document_amd", "csrc", src), "rb").read())
        assert bench.source_sha(k) == h.hexdigest()
    for k, m in bench.MEASURED_TRAFFIC.items():
        t = bench.traffic_bytes(k)
        # figures taken on this source, scaled by the copy calibration; none once the source changed
        if bench.source_sha(k) == m["src"]:
            assert t == m["fetch_kib"] * 1024 * bench.FETCH_FACTOR + m["write_kib"] * 1024 * bench.WRITE_FACTOR
        else:
            assert t is None
    # a stored figure keyed to other sources is stale: reported as null
    fake = {"o_linear": {"src": "0" * 64, "fetch_kib": 1.0, "write_kib": 1.0},
            "merged_attn": {"src": bench.source_sha("merged_attn"), "fetch_kib": 2.0, "write_kib": 3.0}}
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", fake)
    assert bench.traffic_bytes("o_linear") is None
    assert bench.traffic_bytes("merged_attn") == 2.0 * 1024 * bench.FETCH_FACTOR + 3.0 * 1024 * bench.WRITE_FACTOR
    assert bench.traffic_bytes("no_such_kernel") is None


def test_several_gpus_stop_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
