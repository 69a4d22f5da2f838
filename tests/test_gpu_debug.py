"""The debug build (libkalm_debug.so, -DKALM_DEBUG) on the GPU.

Every kernel guards its data-dependent indexes in both builds (the work of a bad
pair is skipped, a bad source row gives NaN).  In the debug build each guard
that fires is also recorded and the entry point returns KALM_ERR_BOUNDS naming
it.  These tests drive each guard with an index the guard itself keeps in
bounds (so no kernel ever accesses memory outside its buffers), check the
status and message of the debug build and the documented skip/NaN result of
the release build, and check that a valid small stack runs through the debug
build with every call OK and the same results as the release build.
"""
import os
import sys

import numpy as np
import pytest
import torch

from encoder_decoder_document_amd import ops, stack, synth
from parity_util import to_dev, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not os.path.exists(ops.DEBUG_LIB_PATH), reason="libkalm_debug.so not built")]


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _expect_bounds(fn, what):
    """fn() through the debug build raises KALM_ERR_BOUNDS naming `what`;
    a valid call right after it is OK again (the record is cleared)."""
    with ops.using(ops.DEBUG_LIB_PATH):
        assert ops.debug_build()
        with pytest.raises(ops.KalmError) as e:
            fn()
        assert e.value.status == ops.KALM_ERR_BOUNDS, str(e.value)
        assert what in str(e.value), str(e.value)


def test_gather_guard():
    _announce("debug gather_rows")
    src = to_dev(synth.normal(50, (37, 256), 1.0, False), torch.float32)
    idx = synth.integers(51, 0, 36, 100)
    good = to_dev(idx, torch.int32)
    idx[7] = 37
    bad = to_dev(idx, torch.int32)
    _expect_bounds(lambda: ops.kalm_gather_rows(src, bad), "gather index")
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = ops.kalm_gather_rows(src, good)
    rel = ops.kalm_gather_rows(src, good)
    torch.cuda.synchronize()
    assert torch.equal(dbg, rel)
    out = ops.kalm_gather_rows(src, bad)   # release: OK, NaN row
    torch.cuda.synchronize()
    assert torch.isnan(out[7]).all() and not torch.isnan(out[:7]).any()


@pytest.mark.parametrize("M,N,bf", [(300, 1152, True), (40003, 1152, True), (33, 20, False)])
def test_residual_source_row_guard(M, N, bf):
    # small-tile path, the big path with the fp32 stream prefetch, the fp32 path
    _announce(f"debug linear_residual M={M} N={N} bf16={bf}")
    K = 1024 if bf else 36
    dt = torch.bfloat16 if bf else torch.float32
    X = to_dev(synth.normal(40, (M, K), 1.0, bf), dt)
    W = to_dev(synth.normal(41, (N, K), 0.02, bf), dt)
    R = to_dev(synth.normal(42, (97, N), 1.0, False), torch.float32)
    idx = synth.integers(43, 0, 96, M)
    good = to_dev(idx, torch.int32)
    idx[M // 2] = 97
    bad = to_dev(idx, torch.int32)
    _expect_bounds(lambda: ops.kalm_linear_residual(X, W, R, bad), "residual source row")
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = ops.kalm_linear_residual(X, W, R, good)
    rel = ops.kalm_linear_residual(X, W, R, good)
    out = ops.kalm_linear_residual(X, W, R, bad)
    torch.cuda.synchronize()
    assert torch.equal(dbg, rel)
    assert torch.isnan(out[M // 2]).all() and not torch.isnan(out[:M // 2]).any()


def _attn_inputs(bf16):
    d = 256 if bf16 else 64
    dt = torch.bfloat16 if bf16 else torch.float32
    nq, nkv, D, Cmax = 4, 1, 3, 40
    lqs = [20, 25, 9]
    rows = sum(lqs)
    Q = to_dev(synth.normal(60, (rows, nq * d), 0.7, bf16), dt)
    Ks = to_dev(synth.normal(61, (rows, nkv * d), 0.7, bf16), dt)
    Vs = to_dev(synth.normal(62, (rows, nkv * d), 1.0, bf16), dt)
    Kc = to_dev(synth.normal(63, (D * Cmax, nkv * d), 0.7, bf16), dt)
    Vc = to_dev(synth.normal(64, (D * Cmax, nkv * d), 1.0, bf16), dt)
    cm = to_dev((np.arange(Cmax)[None] < np.array([[40], [13], [1]])).astype(np.uint8), torch.uint8)
    cu = np.concatenate([[0], np.cumsum(lqs)]).astype(np.int32)
    dop = np.arange(3, dtype=np.int32)
    return Q, Ks, Vs, Kc, Vc, cm, cu, dop, nq, nkv, d


@pytest.mark.parametrize("bf16", [True, False])
def test_attention_guards(bf16):
    _announce(f"debug merged_attn bf16={bf16}")
    Q, Ks, Vs, Kc, Vc, cm, cu, dop, nq, nkv, d = _attn_inputs(bf16)
    run = lambda cu_, dop_: ops.kalm_merged_attn(Q, Ks, Vs, to_dev(cu_, torch.int32), 25, Kc, Vc, cm,
                                                 to_dev(dop_, torch.int32), nq, nkv, d)
    # a passage index outside [0, D)
    bad_dop = dop.copy()
    bad_dop[1] = 3
    _expect_bounds(lambda: run(cu, bad_dop), "passage index")
    # the last pair's rows run past the Q/K/V/O rows (the guard skips the pair)
    bad_cu = cu.copy()
    bad_cu[3] = bad_cu[2] + 25
    _expect_bounds(lambda: run(bad_cu, dop), "pair rows")
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = run(cu, dop)
    rel = run(cu, dop)
    nan_rows = run(cu, bad_dop)
    torch.cuda.synchronize()
    assert torch.equal(dbg, rel)
    g = to_np(nan_rows)
    assert np.isnan(g[20:45]).all() and np.isfinite(g[:20]).all() and np.isfinite(g[45:]).all()


def test_final_row_guard():
    _announce("debug yesno_score")
    h = to_dev(synth.normal(70, (50, 640), 1.0, False), torch.float32)
    w = to_dev(synth.normal(71, (2, 640), 0.02, True), torch.bfloat16)
    fr = synth.integers(72, 0, 49, 9)
    good = to_dev(fr, torch.int32)
    fr[4] = 50
    bad = to_dev(fr, torch.int32)
    _expect_bounds(lambda: ops.kalm_yesno_score(h, bad, w), "final row")
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = ops.kalm_yesno_score(h, good, w)
    rel = ops.kalm_yesno_score(h, good, w)
    s = ops.kalm_yesno_score(h, bad, w)[3]
    torch.cuda.synchronize()
    for a, b in zip(dbg, rel):
        assert torch.equal(a, b)
    assert torch.isnan(s[4]) and not torch.isnan(s[:4]).any()


def test_rope_row_guard():
    _announce("debug rope")
    X = synth.normal(80, (20, 4 * 64), 1.0, False)
    cu_bad = np.array([0, 10, 30], np.int32)   # rows 20..29 do not exist
    cu_good = np.array([0, 10, 20], np.int32)
    Xd = to_dev(X, torch.float32)
    _expect_bounds(lambda: ops.kalm_rope(Xd, 0, 4, 64, to_dev(cu_bad, torch.int32), 20), "RoPE row")
    a, b, c = (to_dev(X, torch.float32) for _ in range(3))
    with ops.using(ops.DEBUG_LIB_PATH):
        ops.kalm_rope(a, 0, 4, 64, to_dev(cu_good, torch.int32), 10)
    ops.kalm_rope(b, 0, 4, 64, to_dev(cu_good, torch.int32), 10)
    ops.kalm_rope(c, 0, 4, 64, to_dev(cu_bad, torch.int32), 20)  # release: in-range rows only
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(c, b)


def test_layout_overflow_guard():
    _announce("debug pair_layout overflow")
    lq = to_dev(np.array([1 << 29, (1 << 29) - 3, 5], np.int32), torch.int32)
    _expect_bounds(lambda: ops.kalm_pair_layout(lq, 3, with_h0_row=False), "INT32_MAX")
    ok = to_dev(np.array([3, 1, 4], np.int32), torch.int32)
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = ops.kalm_pair_layout(ok, 5, rows=40)
    rel = ops.kalm_pair_layout(ok, 5, rows=40)
    torch.cuda.synchronize()
    for k in dbg:
        assert torch.equal(dbg[k], rel[k]), k


@pytest.mark.parametrize("shape_index", [0, 1])
def test_valid_stack_is_clean_and_identical(shape_index):
    """A whole step through the debug build: no guard fires, and every output
    equals the release build's (the kernels differ only by the records)."""
    _announce(f"debug stack shape {shape_index}")
    inp = synth.make_inputs(shape_index)
    b = stack.upload(inp, device="cuda:0")
    rel = [t.clone() for t in stack.step(b)]
    with ops.using(ops.DEBUG_LIB_PATH):
        dbg = [t.clone() for t in stack.step(b)]
    torch.cuda.synchronize()
    for a, c in zip(dbg, rel):
        assert torch.equal(a, c)
