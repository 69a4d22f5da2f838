"""Guard regions around every output of every entry point (GPU).

Each output buffer is a view into a larger allocation with 4 KiB before and
after it; the whole allocation, view included, is first filled with a canary
bit pattern (a NaN payload for floating types, 0xA5 bytes for masks, a large
sentinel for indexes).  After the call the guard regions must still hold the
canary -- no kernel writes outside its output -- and, where the entry point
writes every output element, no element of the view may still hold it.  The
shapes are ragged (partial tiles at every edge) and cover the tile paths of
the GEMM (small tiles, 128 x 128 with a row mask or the fp32 stream, the
persistent 256 x 256 kernel).  Outputs are also compared with the same call
into plain, unguarded tensors.
"""
import math
import sys

import numpy as np
import pytest
import torch

from encoder_decoder_document_amd import ops, synth
from parity_util import to_dev

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096
_INT_VIEW = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
_CANARY = {1: 0xA5, 2: 0x7FA5, 4: 0x7FA5A5A5}


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


class Guarded:
    """A device tensor of `shape` inside guard regions, all of it canary-filled."""

    def __init__(self, shape, dtype):
        self.el = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // self.el
        self.n = math.prod(shape)
        self.buf = torch.empty(2 * self.g + self.n, dtype=dtype, device="cuda")
        self.ints().fill_(_CANARY[self.el])
        self.t = self.buf[self.g:self.g + self.n].view(shape)

    def ints(self, t=None):
        return (self.buf if t is None else t).view(_INT_VIEW[self.el])

    def check(self, name, written=True):
        torch.cuda.synchronize()
        ib = self.ints()
        c = _CANARY[self.el]
        assert bool((ib[:self.g] == c).all()), f"{name}: write before the output"
        assert bool((ib[self.g + self.n:] == c).all()), f"{name}: write after the output"
        if written:
            left = int((ib[self.g:self.g + self.n] == c).sum())
            assert left == 0, f"{name}: {left} of {self.n} elements not written"


def _same(a, b, name):
    torch.cuda.synchronize()
    assert torch.equal(a.view(_INT_VIEW[a.element_size()]), b.view(_INT_VIEW[b.element_size()])), name


def test_pair_layout_guarded():
    _announce("canary pair_layout")
    lq = np.array([3, 1, 64, 7, 1], np.int32)
    D = 37
    P, rows = len(lq) * D, int(D * lq.sum())
    outs = {k: Guarded((n,), torch.int32) for k, n in
            (("cu_q", P + 1), ("doc", P), ("fin", P), ("h0", rows), ("h0f", P), ("cu_u", len(lq) + 1))}
    st = ops.load().kalm_pair_layout(to_dev(lq, torch.int32).data_ptr(), len(lq), D, outs["cu_q"].t.data_ptr(),
                                     outs["doc"].t.data_ptr(), outs["fin"].t.data_ptr(), outs["h0"].t.data_ptr(),
                                     rows, outs["h0f"].t.data_ptr(), outs["cu_u"].t.data_ptr(), None)
    assert st == ops.KALM_OK
    for k, o in outs.items():
        o.check(f"pair_layout {k}")
    ref = ops.kalm_pair_layout(to_dev(lq, torch.int32), D, rows=rows)
    for k, rk in (("cu_q", "cu_q"), ("doc", "doc_of_pair"), ("fin", "final_row"), ("h0", "h0_row"),
                  ("h0f", "h0_final"), ("cu_u", "cu_u")):
        _same(outs[k].t, ref[rk], k)


@pytest.mark.parametrize("D,T,H,chunk,bf16", [(7, 37, 640, 4, True), (5, 130, 1152, 3, False)])
def test_chunk_pool_guarded(D, T, H, chunk, bf16):
    _announce(f"canary chunk_pool D={D} T={T} H={H} chunk={chunk}")
    dt = torch.bfloat16 if bf16 else torch.float32
    x = to_dev(synth.normal(1, (D, T, H), 1.0, bf16), dt)
    lens = synth.integers(2, 0, T, D)
    m = to_dev((np.arange(T)[None] < lens[:, None]).astype(np.uint8), torch.uint8)
    C = -(-T // chunk)
    o = (Guarded((D, C, H), dt), Guarded((D, C), torch.uint8), Guarded((D,), torch.int32))
    ops.kalm_chunk_pool(x, m, chunk, out=tuple(g.t for g in o))
    for g, k in zip(o, ("pooled", "chunk_mask", "n_chunks")):
        g.check(f"chunk_pool {k}")
    ref = ops.kalm_chunk_pool(x, m, chunk)
    for g, r, k in zip(o, ref, ("pooled", "chunk_mask", "n_chunks")):
        _same(g.t, r, k)


@pytest.mark.parametrize("D,C,H,kv,L", [(7, 37, 640, 256, 1), (50, 256, 1152, 256, 6)])
def test_cross_kv_guarded(D, C, H, kv, L):
    # L = 6 at D = 50: the row-masked 128 x 128 path of the big GEMM
    _announce(f"canary cross_kv_layers D={D} C={C} L={L}")
    pooled = to_dev(synth.normal(3, (D, C, H), 1.0, True), torch.bfloat16)
    cm = to_dev(synth.bernoulli_mask(4, 0.6, (D, C)), torch.uint8)
    W = to_dev(synth.normal(5, (L, 2 * kv, H), 0.02, True), torch.bfloat16)
    o = Guarded((D, C, L, 2 * kv), torch.bfloat16)
    ops.kalm_cross_kv_layers(pooled, cm, W, out=o.t)
    o.check("cross_kv_layers")
    _same(o.t, ops.kalm_cross_kv_layers(pooled, cm, W), "cross_kv_layers")
    if L == 1:
        o1 = Guarded((D, C, 2 * kv), torch.bfloat16)
        ops.kalm_cross_kv(pooled, cm, W[0], out=o1.t)
        o1.check("cross_kv")
        _same(o1.t, o.t.view(D, C, 2 * kv), "cross_kv")


@pytest.mark.parametrize("M,K,N,mode", [(1000, 1152, 1536, "bf16"), (22093, 1152, 1536, "bf16"),
                                        (333, 1024, 1160, "f32"), (301, 1024, 1152, "acc"),
                                        (40003, 1024, 1152, "acc"), (77, 36, 20, "f32in")])
def test_linear_guarded(M, K, N, mode):
    # small tiles; the persistent 256 x 256 kernel; fp32 output; accumulate on the
    # small and on the 128 x 128 fp32-stream path (with the bf16 copy); fp32 inputs
    _announce(f"canary linear M={M} K={K} N={N} {mode}")
    bf = mode != "f32in"
    dt = torch.bfloat16 if bf else torch.float32
    X = to_dev(synth.normal(10, (M, K), 1.0, bf), dt)
    W = to_dev(synth.normal(11, (N, K), 0.02, bf), dt)
    ydt = torch.bfloat16 if mode == "bf16" else torch.float32
    Y = Guarded((M, N), ydt)
    Yb = Guarded((M, N), torch.bfloat16) if mode == "acc" else None
    Yref = torch.empty(M, N, dtype=ydt, device="cuda")
    if mode == "acc":
        start = to_dev(synth.normal(12, (M, N), 1.0, False), torch.float32)
        Y.t.copy_(start)
        Yref.copy_(start)
    ops.kalm_linear(X, W, Y.t, accumulate=mode == "acc", Y_bf16=Yb.t if Yb else None)
    Y.check("linear Y")
    if Yb:
        Yb.check("linear Y_bf16")
    Ybr = torch.empty(M, N, dtype=torch.bfloat16, device="cuda") if Yb else None
    ops.kalm_linear(X, W, Yref, accumulate=mode == "acc", Y_bf16=Ybr)
    _same(Y.t, Yref, "Y")
    if Yb:
        _same(Yb.t, Ybr, "Y_bf16")


@pytest.mark.parametrize("M,N", [(300, 1152), (40003, 1160)])
def test_linear_residual_guarded(M, N):
    _announce(f"canary linear_residual M={M} N={N}")
    K = 1024
    X = to_dev(synth.normal(20, (M, K), 1.0, True), torch.bfloat16)
    W = to_dev(synth.normal(21, (N, K), 0.02, True), torch.bfloat16)
    R = to_dev(synth.normal(22, (97, N), 1.0, False), torch.float32)
    idx = to_dev(synth.integers(23, 0, 96, M), torch.int32)
    Y, Yb = Guarded((M, N), torch.float32), Guarded((M, N), torch.bfloat16)
    ops.kalm_linear_residual(X, W, R, idx, Y=Y.t, Y_bf16=Yb.t)
    Y.check("residual Y")
    Yb.check("residual Y_bf16")
    Yr = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    _same(Y.t, ops.kalm_linear_residual(X, W, R, idx, Y_bf16=Yr), "Y")
    _same(Yb.t, Yr, "Y_bf16")


def test_gather_rows_guarded():
    _announce("canary gather_rows")
    src = to_dev(synth.normal(30, (37, 1160), 1.0, False), torch.float32)
    idx = to_dev(synth.integers(31, 0, 36, 501), torch.int32)
    d, db = Guarded((501, 1160), torch.float32), Guarded((501, 1160), torch.bfloat16)
    ops.kalm_gather_rows(src, idx, dst=d.t, dst_bf16=db.t)
    d.check("gather dst")
    db.check("gather dst_bf16")
    _same(d.t, ops.kalm_gather_rows(src, idx), "dst")


def _attn(bf16, lqs=(1, 33, 64, 130, 7), D=3, Cmax=77):
    d = 256 if bf16 else 64
    dt = torch.bfloat16 if bf16 else torch.float32
    nq, nkv = 4, 1
    rows = sum(lqs)
    P = len(lqs)
    Q = to_dev(synth.normal(40, (rows, nq * d), 0.7, bf16), dt)
    Ks = to_dev(synth.normal(41, (rows, nkv * d), 0.7, bf16), dt)
    Vs = to_dev(synth.normal(42, (rows, nkv * d), 1.0, bf16), dt)
    Kc = to_dev(synth.normal(43, (D * Cmax, nkv * d), 0.7, bf16), dt)
    Vc = to_dev(synth.normal(44, (D * Cmax, nkv * d), 1.0, bf16), dt)
    cm = to_dev(synth.bernoulli_mask(45, 0.5, (D, Cmax)), torch.uint8)
    cu = to_dev(np.concatenate([[0], np.cumsum(lqs)]).astype(np.int32), torch.int32)
    dop = to_dev((np.arange(P) % D).astype(np.int32), torch.int32)
    return dict(Q=Q, Ks=Ks, Vs=Vs, Kc=Kc, Vc=Vc, cm=cm, cu=cu, dop=dop, nq=nq, nkv=nkv, d=d, rows=rows, P=P,
                max_lq=max(lqs), dt=dt)


@pytest.mark.parametrize("bf16", [True, False])
def test_merged_attn_guarded(bf16):
    _announce(f"canary merged_attn bf16={bf16}")
    a = _attn(bf16)
    O, L = Guarded((a["rows"], a["nq"] * a["d"]), a["dt"]), Guarded((a["rows"], a["nq"]), torch.float32)
    args = (a["Q"], a["Ks"], a["Vs"], a["cu"], a["max_lq"], a["Kc"], a["Vc"], a["cm"], a["dop"], a["nq"], a["nkv"],
            a["d"])
    ops.kalm_merged_attn(*args, out=O.t, lse=L.t)
    O.check("merged_attn O")
    L.check("merged_attn lse")
    _same(O.t, ops.kalm_merged_attn(*args), "O")
    # final rows only: one output row per pair
    Of, Lf = Guarded((a["P"], a["nq"] * a["d"]), a["dt"]), Guarded((a["P"], a["nq"]), torch.float32)
    ops.kalm_merged_attn_rows(*args, row_mode=ops.ROWS_FINAL, o_rows=a["P"], out=Of.t, lse=Lf.t)
    Of.check("merged_attn_rows O")
    Lf.check("merged_attn_rows lse")


@pytest.mark.parametrize("bf16", [True, False])
def test_self_partial_and_resume_guarded(bf16):
    _announce(f"canary self partial / resume / split bf16={bf16}")
    a = _attn(bf16)
    rows, nq, d = a["rows"], a["nq"], a["d"]
    Os, Ls = Guarded((rows, nq * d), torch.float32), Guarded((rows, nq), torch.float32)
    ops.kalm_self_attn_partial(a["Q"], a["Ks"], a["Vs"], a["cu"], a["max_lq"], nq, a["nkv"], d, out=Os.t, lse=Ls.t)
    Os.check("self partial O")
    Ls.check("self partial lse")
    rargs = (a["Q"], Os.t, Ls.t, a["cu"], a["max_lq"], a["Kc"], a["Vc"], a["cm"], a["dop"], nq, a["nkv"], d,
             ops.ROWS_ALL, rows)
    Or, Lr = Guarded((rows, nq * d), a["dt"]), Guarded((rows, nq), torch.float32)
    ops.kalm_merged_attn_resume(*rargs, out=Or.t, lse=Lr.t)
    Or.check("resume O")
    Lr.check("resume lse")
    if bf16:
        ws = Guarded((ops.split_workspace_bytes(3, rows, nq, d),), torch.uint8)
        Osp = Guarded((rows, nq * d), a["dt"])
        ops.kalm_merged_attn_split(*rargs, n_split=3, workspace=ws.t, out=Osp.t)
        ws.check("split workspace", written=False)
        Osp.check("split O")
        Ona = Guarded((rows, nq * d), a["dt"])
        ops.kalm_merged_attn_split_noalloc(*rargs, n_split=3, out=Ona.t)
        Ona.check("split noalloc O")
        _same(Ona.t, Osp.t, "noalloc O")


def test_layer_parts_guarded():
    _announce("canary rms_norm / rope / gated gelu")
    M, H, I = 333, 1152, 768
    x = to_dev(synth.normal(50, (M, H), 1.0, False), torch.float32)
    w = to_dev(synth.normal(51, (H,), 1.0, True), torch.bfloat16)
    y = Guarded((M, H), torch.bfloat16)
    ops.kalm_rms_norm(x, w, out=y.t)
    y.check("rms_norm")
    _same(y.t, ops.kalm_rms_norm(x, w, y_dtype=torch.bfloat16), "rms_norm")
    # RoPE rotates in place: the guards around X must hold, X itself is input
    lens = np.array([1, 31, 130, 7], np.int32)
    cu = to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), torch.int32)
    rows = int(lens.sum())
    X = Guarded((rows, 6 * 256), torch.bfloat16)
    X.t.copy_(to_dev(synth.normal(52, (rows, 6 * 256), 1.0, True), torch.bfloat16))
    ops.kalm_rope(X.t, 0, 4, 256, cu, int(lens.max()))
    X.check("rope", written=False)
    Y = to_dev(synth.normal(53, (M, 2 * I), 1.0, True), torch.bfloat16)
    A = Guarded((M, I), torch.bfloat16)
    ops.kalm_gated_gelu(Y, out=A.t)
    A.check("gated_gelu")
    Xg = to_dev(synth.normal(54, (1100, H), 1.0, True), torch.bfloat16)
    Wg = to_dev(synth.normal(55, (I, H), 0.02, True), torch.bfloat16)
    Wu = to_dev(synth.normal(56, (I, H), 0.02, True), torch.bfloat16)
    A2 = Guarded((1100, I), torch.bfloat16)
    ops.kalm_linear_gated_gelu(Xg, Wg, Wu, out=A2.t)
    A2.check("linear_gated_gelu")
    _same(A2.t, ops.kalm_linear_gated_gelu(Xg, Wg, Wu), "linear_gated_gelu")


def test_score_and_rank_guarded():
    _announce("canary yesno / rank_topn")
    lib = ops.load()
    h = to_dev(synth.normal(60, (300, 1152), 1.0, False), torch.float32)
    w = to_dev(synth.normal(61, (2, 1152), 0.02, True), torch.bfloat16)
    fr = to_dev(synth.integers(62, 0, 299, 57), torch.int32)
    outs = [Guarded((57,), torch.float32) for _ in range(4)]
    st = lib.kalm_yesno_score(h.data_ptr(), ops.KALM_F32, 1152, 300, fr.data_ptr(), 57, 1152, w.data_ptr(),
                              ops.KALM_BF16, *[o.t.data_ptr() for o in outs], None)
    assert st == ops.KALM_OK
    for o, k in zip(outs, ("yes", "no", "margin", "score")):
        o.check(f"yesno {k}")
    for o, r in zip(outs, ops.kalm_yesno_score(h, fr, w)):
        _same(o.t, r, "yesno")
    score = to_dev(synth.normal(63, (3, 100), 1.0, False), torch.float32)
    gi, gv = Guarded((3, 10), torch.int32), Guarded((3, 10), torch.float32)
    st = lib.kalm_rank_topn(score.data_ptr(), 3, 100, 10, gi.t.data_ptr(), gv.t.data_ptr(), None)
    assert st == ops.KALM_OK
    gi.check("rank index")
    gv.check("rank score")
    ri, rv = ops.kalm_rank_topn(score, 10)
    _same(gi.t, ri, "rank index")
    _same(gv.t, rv, "rank score")
